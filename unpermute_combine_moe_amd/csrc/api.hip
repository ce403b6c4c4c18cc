// C ABI of libmoeperm: host-side argument checks, then the launchers.
// Every check runs before anything is enqueued; see include/libmoeperm.h for
// the contract of each call.
#include "libmoeperm.h"

#include <limits.h>

#include <algorithm>

#include "launch.hpp"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int32_t kAbiVersion = 3;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
// a row tensor: non-null and 16-byte aligned
inline bool row_ok(const void* p) { return p != nullptr && aligned(p, 16); }
// an int32 / fp32 tensor: non-null and 4-byte aligned
inline bool word_ok(const void* p) { return p != nullptr && aligned(p, 4); }

inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

const uint16_t* u16(const void* p) { return static_cast<const uint16_t*>(p); }
uint16_t* u16(void* p) { return static_cast<uint16_t*>(p); }

moe_status_t check_tk(int64_t T, int32_t K) {
  if (T < 0 || K < 1 || K > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (T * int64_t(K) > INT32_MAX) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_h(int32_t H) {
  if (H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The special-expert block of the combine and its backward ([CV2] 参数说明:
// ori_x is required by copy and const experts, alpha and v by const ones;
// 约束说明: all expert ids must stay below 2^31 - 1).
moe_status_t parse_special(const moe_special_experts_t* special, int32_t num_experts, int64_t T,
                           moe::SpecialArgs* sp) {
  *sp = moe::SpecialArgs{0, 0, 0, nullptr, nullptr, nullptr, 0, 0, 0, nullptr};
  if (special == nullptr) return MOE_OK;
  if (special->num_zero < 0 || special->num_copy < 0 || special->num_const < 0)
    return MOE_ERR_INVALID_ARG;
  const int64_t ids_total =
      int64_t(num_experts) + special->num_zero + special->num_copy + special->num_const;
  if (ids_total >= INT32_MAX) return MOE_ERR_INVALID_ARG;
  sp->num_zero = special->num_zero;
  sp->num_copy = special->num_copy;
  sp->num_const = special->num_const;
  if (sp->num_copy + sp->num_const > 0) {
    if (T > 0 && !row_ok(special->ori_x)) return MOE_ERR_INVALID_ARG;
    sp->ori_x = u16(special->ori_x);
  }
  if (sp->num_const > 0) {
    if (!word_ok(special->alpha1) || !word_ok(special->alpha2) || !row_ok(special->const_v))
      return MOE_ERR_INVALID_ARG;
    sp->alpha1 = special->alpha1;
    sp->alpha2 = special->alpha2;
    sp->a_st = special->alpha_stride_t;
    sp->a_sc = special->alpha_stride_c;
    sp->a_sh = special->alpha_stride_h;
    sp->const_v = u16(special->const_v);
  }
  return MOE_OK;
}

}  // namespace

MOE_API const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

MOE_API int32_t moe_abi_version(void) { return kAbiVersion; }

// --------------------------------------------------------------------------- permute

MOE_API moe_status_t moe_permute_workspace_size(int64_t T, int32_t K, int32_t E, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (moe_status_t s = check_tk(T, K)) return s;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  *bytes = moe::permute_workspace_bytes(T, K, E);
  return MOE_OK;
}

MOE_API moe_status_t moe_permute(const void* x, const int32_t* expert_ids,
                                 const uint8_t* active_mask, int32_t mask_per_slot, int64_t T,
                                 int32_t H, int32_t K, int32_t num_experts, void* permuted,
                                 int32_t* sorted_slot, int32_t* row_of_slot,
                                 int32_t* expert_counts, int32_t* expert_offsets, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (permuted != nullptr) {
    if (moe_status_t s = check_h(H)) return s;
  }
  if (!word_ok(expert_counts) || !word_ok(expert_offsets)) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!word_ok(expert_ids) || !word_ok(sorted_slot) || !word_ok(row_of_slot))
      return MOE_ERR_INVALID_ARG;
    if (permuted != nullptr && (!row_ok(x) || !row_ok(permuted))) return MOE_ERR_INVALID_ARG;
  }
  if (mask_per_slot != 0 && mask_per_slot != 1) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::permute_workspace_bytes(T, K, num_experts);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
    return MOE_ERR_WORKSPACE;
  const moe::SlotMask mk{active_mask, mask_per_slot, K};
  return hip_status(moe::launch_permute(u16(x), expert_ids, mk, T, H, K, num_experts, u16(permuted),
                                        sorted_slot, row_of_slot, expert_counts, expert_offsets,
                                        workspace, stream));
}

MOE_API moe_status_t moe_permute_rows(const void* x, const int32_t* row_of_slot, int64_t T,
                                      int32_t H, int32_t K, int64_t N, void* permuted,
                                      hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (moe_status_t s = check_h(H)) return s;
  if (N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!row_ok(x) || !word_ok(row_of_slot))) return MOE_ERR_INVALID_ARG;
  if (N > 0 && !row_ok(permuted)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_permute_rows(u16(x), row_of_slot, T, H, K, N, u16(permuted),
                                             stream));
}

// --------------------------------------------------------------------------- reorder

MOE_API moe_status_t moe_rank_to_expert_reorder_workspace_size(int32_t R, int32_t E_local,
                                                               size_t* bytes) {
  if (bytes == nullptr || R < 1 || E_local < 1 ||
      int64_t(R) * E_local > MOE_MAX_REORDER_BLOCKS)
    return MOE_ERR_INVALID_ARG;
  *bytes = moe::reorder_workspace_bytes(R, E_local);
  return MOE_OK;
}

MOE_API moe_status_t moe_rank_to_expert_reorder(const void* x_rank_major, const int32_t* counts,
                                                int32_t R, int32_t E_local, int64_t N, int32_t H,
                                                void* y_expert_major, int32_t* perm,
                                                int32_t* inv_perm, int32_t* tokens_per_expert,
                                                int32_t* expert_offsets, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
  if (R < 1 || E_local < 1 || int64_t(R) * E_local > MOE_MAX_REORDER_BLOCKS)
    return MOE_ERR_INVALID_ARG;
  if (N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if ((x_rank_major == nullptr) != (y_expert_major == nullptr)) return MOE_ERR_INVALID_ARG;
  if (y_expert_major != nullptr) {
    if (moe_status_t s = check_h(H)) return s;
    if (N > 0 && (!row_ok(x_rank_major) || !row_ok(y_expert_major))) return MOE_ERR_INVALID_ARG;
  }
  if (!word_ok(counts) || !word_ok(tokens_per_expert) || !word_ok(expert_offsets))
    return MOE_ERR_INVALID_ARG;
  if (N > 0 && !word_ok(perm)) return MOE_ERR_INVALID_ARG;
  if (inv_perm != nullptr && !aligned(inv_perm, 4)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::reorder_workspace_bytes(R, E_local);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_reorder(u16(x_rank_major), counts, R, E_local, N, H,
                                        u16(y_expert_major), perm, inv_perm, tokens_per_expert,
                                        expert_offsets, workspace, stream));
}

// --------------------------------------------------------------------------- grouped GEMM

namespace {
// Largest H and I: the GEMM epilogue addresses one 128-row output tile (at most
// 128 x 2I or 128 x H bf16) with 32-bit byte offsets below 2^31.
constexpr int32_t kMaxGemmDim = 1 << 20;

moe_status_t check_gemm_sizes(int32_t E, int64_t N_cap, int32_t H, int32_t I) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (N_cap < 0 || N_cap > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (H > kMaxGemmDim || I > kMaxGemmDim) return MOE_ERR_UNSUPPORTED;
  // the kernel indexes (row tile, column tile) pairs with 32-bit integers
  const int64_t max_row_tiles = N_cap / 128 + E + 1;
  const int64_t max_col_tiles = (std::max(H, I) + 127) / 128;
  if (max_row_tiles * max_col_tiles >= INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

MOE_API moe_status_t moe_grouped_gemm_swiglu_workspace_size(int32_t E, int64_t N_cap, int32_t H,
                                                            int32_t I, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (moe_status_t s = check_gemm_sizes(E, N_cap, H, I)) return s;
  *bytes = moe::gemm_workspace_bytes(E, N_cap, H, I);
  return MOE_OK;
}

MOE_API moe_status_t moe_grouped_gemm_swiglu(const void* x, const int32_t* expert_offsets,
                                             int32_t E, int64_t N_cap, int32_t H, int32_t I,
                                             const void* w_gate, const void* w_up,
                                             const void* w_down, void* h, void* y,
                                             float* preact, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  if (moe_status_t s = check_gemm_sizes(E, N_cap, H, I)) return s;
  if (!word_ok(expert_offsets)) return MOE_ERR_INVALID_ARG;
  if (!row_ok(w_gate) || !row_ok(w_up) || !row_ok(w_down)) return MOE_ERR_INVALID_ARG;
  if (N_cap > 0 && (!row_ok(x) || !row_ok(h) || !row_ok(y))) return MOE_ERR_INVALID_ARG;
  if (preact != nullptr && !aligned(preact, 16)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::gemm_workspace_bytes(E, N_cap, H, I);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_grouped_gemm_swiglu(u16(x), expert_offsets, E, N_cap, H, I,
                                                    u16(w_gate), u16(w_up), u16(w_down), u16(h),
                                                    u16(y), N_cap > 0 ? preact : nullptr,
                                                    workspace, stream));
}

MOE_API moe_status_t moe_grouped_gemm_swiglu_grad_workspace_size(int32_t E, int64_t N_cap,
                                                                 int32_t H, int32_t I,
                                                                 size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > MOE_MAX_EXPERTS || N_cap < 0 || N_cap > INT32_MAX || H <= 0 || I <= 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (H > kMaxGemmDim || I > kMaxGemmDim) return MOE_ERR_UNSUPPORTED;
  *bytes = moe::gemm_grad_workspace_bytes(E, N_cap, H, I);
  return MOE_OK;
}

MOE_API moe_status_t moe_grouped_gemm_swiglu_grad(
    const void* x, const int32_t* expert_offsets, int32_t E, int64_t N_cap, int32_t H, int32_t I,
    const void* w_gate, const void* w_up, const void* w_down, const void* h, const void* dy,
    void* dx, void* dw_gate, void* dw_up, void* dw_down, const float* preact, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || N_cap < 0 || N_cap > INT32_MAX || H <= 0 || I <= 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (H > kMaxGemmDim || I > kMaxGemmDim) return MOE_ERR_UNSUPPORTED;
  if (!word_ok(expert_offsets) || !row_ok(w_gate) || !row_ok(w_up) || !row_ok(w_down) ||
      !row_ok(dw_gate) || !row_ok(dw_up) || !row_ok(dw_down))
    return MOE_ERR_INVALID_ARG;
  if (N_cap > 0 && (!row_ok(x) || !row_ok(h) || !row_ok(dy) || !row_ok(dx)))
    return MOE_ERR_INVALID_ARG;
  if (preact != nullptr && !aligned(preact, 16)) return MOE_ERR_INVALID_ARG;
  if (workspace == nullptr || !aligned(workspace, 256) ||
      workspace_bytes < moe::gemm_grad_workspace_bytes(E, N_cap, H, I))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_grouped_gemm_swiglu_grad(
      u16(x), expert_offsets, E, N_cap, H, I, u16(w_gate), u16(w_up), u16(w_down), u16(h), u16(dy),
      u16(dx), u16(dw_gate), u16(dw_up), u16(dw_down), N_cap > 0 ? preact : nullptr, workspace,
      stream));
}

// --------------------------------------------------------------------------- combine

MOE_API moe_status_t moe_unpermute_combine(const void* expert_out, int64_t N,
                                           const int32_t* row_of_slot, const int32_t* row_map,
                                           const int32_t* expert_ids, const float* probs,
                                           const uint8_t* active_mask, int32_t mask_per_slot,
                                           int64_t T, int32_t K, int32_t H, int32_t num_experts,
                                           const moe_special_experts_t* special,
                                           const void* shared_x, void* out, hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (moe_status_t s = check_h(H)) return s;
  if (num_experts < 1 || N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  moe::SpecialArgs sp;
  if (moe_status_t s = parse_special(special, num_experts, T, &sp)) return s;
  if (T > 0) {
    if (!word_ok(row_of_slot) || !word_ok(expert_ids) || !word_ok(probs) || !row_ok(out))
      return MOE_ERR_INVALID_ARG;
    if (N > 0 && !row_ok(expert_out)) return MOE_ERR_INVALID_ARG;
    if (row_map != nullptr && !aligned(row_map, 4)) return MOE_ERR_INVALID_ARG;
    if (shared_x != nullptr && !aligned(shared_x, 16)) return MOE_ERR_INVALID_ARG;
  }
  if (mask_per_slot != 0 && mask_per_slot != 1) return MOE_ERR_INVALID_ARG;
  const moe::SlotMask mk{active_mask, mask_per_slot, K};
  return hip_status(moe::launch_combine(u16(expert_out), N, row_of_slot, row_map, expert_ids,
                                        probs, mk, T, K, H, num_experts, sp, u16(shared_x), u16(out),
                                        stream));
}

// --------------------------------------------------------------------------- backward

MOE_API moe_status_t moe_permute_grad(const void* d_permuted, int64_t N,
                                      const int32_t* row_of_slot, int64_t T, int32_t K, int32_t H,
                                      void* d_x, hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (moe_status_t s = check_h(H)) return s;
  if (N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!word_ok(row_of_slot) || !row_ok(d_x)) return MOE_ERR_INVALID_ARG;
    if (N > 0 && !row_ok(d_permuted)) return MOE_ERR_INVALID_ARG;
  }
  return hip_status(moe::launch_permute_grad(u16(d_permuted), N, row_of_slot, T, K, H, u16(d_x),
                                             stream));
}

MOE_API moe_status_t moe_unpermute_combine_grad_workspace_size(int64_t T, int32_t H,
                                                              int32_t num_const, size_t* bytes) {
  if (bytes == nullptr || T < 0 || T > INT32_MAX || num_const < 0) return MOE_ERR_INVALID_ARG;
  if (moe_status_t s = check_h(H)) return s;
  *bytes = moe::combine_grad_workspace_bytes(T, H, num_const);
  return MOE_OK;
}

MOE_API moe_status_t moe_unpermute_combine_grad(
    const void* grad_out, const void* expert_out, int64_t N, const int32_t* row_of_slot,
    const int32_t* row_map, const int32_t* expert_ids, const float* probs,
    const uint8_t* active_mask, int32_t mask_per_slot, int64_t T, int32_t K, int32_t H,
    int32_t num_experts, const moe_special_experts_t* special, void* d_expert_out,
    float* d_probs, void* d_ori_x, float* d_alpha1, float* d_alpha2, void* d_const_v,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (moe_status_t s = check_h(H)) return s;
  if (num_experts < 1 || N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  moe::SpecialArgs sp;
  if (moe_status_t s = parse_special(special, num_experts, T, &sp)) return s;
  const bool want_alpha = d_alpha1 != nullptr || d_alpha2 != nullptr;
  if (T > 0) {
    if (!row_ok(grad_out) || !word_ok(row_of_slot) || !word_ok(expert_ids) || !word_ok(probs) ||
        !word_ok(d_probs))
      return MOE_ERR_INVALID_ARG;
    if (N > 0 && !row_ok(expert_out)) return MOE_ERR_INVALID_ARG;
    if (row_map != nullptr && !aligned(row_map, 4)) return MOE_ERR_INVALID_ARG;
    if (d_expert_out != nullptr && !aligned(d_expert_out, 16)) return MOE_ERR_INVALID_ARG;
    if (d_ori_x != nullptr && !aligned(d_ori_x, 16)) return MOE_ERR_INVALID_ARG;
    if (d_const_v != nullptr && !aligned(d_const_v, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(d_alpha1, 4) || !aligned(d_alpha2, 4)) return MOE_ERR_INVALID_ARG;
  }
  if (mask_per_slot != 0 && mask_per_slot != 1) return MOE_ERR_INVALID_ARG;
  const moe::AlphaLayout lay = moe::classify_alpha(sp, H);
  if (want_alpha && lay == moe::AlphaLayout::kOther) return MOE_ERR_UNSUPPORTED;
  const bool cross_token =
      sp.num_const > 0 && (d_const_v != nullptr ||
                           (want_alpha && (lay == moe::AlphaLayout::kSharedAlongH ||
                                           lay == moe::AlphaLayout::kSharedScalar)));
  if (T > 0 && cross_token) {
    if (workspace == nullptr || !aligned(workspace, 16) ||
        workspace_bytes < moe::combine_grad_workspace_bytes(T, H, sp.num_const))
      return MOE_ERR_WORKSPACE;
  }
  const moe::SlotMask mk{active_mask, mask_per_slot, K};
  const moe::CombineGradArgs o{u16(d_expert_out), d_probs, u16(d_ori_x), d_alpha1, d_alpha2,
                               u16(d_const_v)};
  return hip_status(moe::launch_combine_grad(u16(grad_out), u16(expert_out), N, row_of_slot,
                                             row_map, expert_ids, probs, mk, T, K, H, num_experts,
                                             sp,
                                             o, workspace, stream));
}

MOE_API moe_status_t moe_unpermute_grad(const void* grad_out, const void* permuted, int64_t N,
                                        const int32_t* row_of_slot, const float* probs,
                                        int64_t T, int32_t K, int32_t H, void* d_permuted,
                                        float* d_probs, hipStream_t stream) {
  if (moe_status_t s = check_tk(T, K)) return s;
  if (moe_status_t s = check_h(H)) return s;
  if (N < 0 || N > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!row_ok(grad_out) || !word_ok(row_of_slot) || !word_ok(probs) || !word_ok(d_probs))
      return MOE_ERR_INVALID_ARG;
    if (N > 0 && (!row_ok(permuted) || !row_ok(d_permuted))) return MOE_ERR_INVALID_ARG;
  }
  return hip_status(moe::launch_unpermute_grad(u16(grad_out), u16(permuted), N, row_of_slot,
                                               probs, T, K, H, u16(d_permuted), d_probs, stream));
}

// --------------------------------------------------------------------------- deredundency

namespace {

moe_status_t check_dered(int32_t oep, int32_t E, int32_t expert_start, int32_t iep, int32_t El) {
  if (oep < 1 || E < 1 || iep < 1 || El < 1 || expert_start < 0) return MOE_ERR_INVALID_ARG;
  if (int64_t(oep) * E > MOE_MAX_DERED_CELLS) return MOE_ERR_INVALID_ARG;
  if (int64_t(iep) * El > E || int64_t(expert_start) + int64_t(iep) * El > E)
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status_t moe_deredundency_dispatch_indices_workspace_size(int32_t oep_size,
                                                                      int32_t num_experts,
                                                                      int32_t iep_size,
                                                                      int32_t num_local_experts,
                                                                      size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (moe_status_t s = check_dered(oep_size, num_experts, 0, iep_size, num_local_experts))
    return s;
  *bytes = moe::dered_indices_workspace_bytes(oep_size, num_experts, iep_size, num_local_experts);
  return MOE_OK;
}

MOE_API moe_status_t moe_deredundency_dispatch_indices(
    const int32_t* tokens_per_expert_by_source, int32_t oep_size, int32_t num_experts,
    int32_t expert_start, int32_t iep_size, int32_t num_local_experts, int64_t capacity,
    int32_t* indices, int32_t* counts_by_dest, int32_t* total, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (moe_status_t s =
          check_dered(oep_size, num_experts, expert_start, iep_size, num_local_experts))
    return s;
  if (capacity < 0 || capacity > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!word_ok(tokens_per_expert_by_source) || !word_ok(counts_by_dest))
    return MOE_ERR_INVALID_ARG;
  if (capacity > 0 && !word_ok(indices)) return MOE_ERR_INVALID_ARG;
  if (total != nullptr && !aligned(total, 4)) return MOE_ERR_INVALID_ARG;
  const size_t need =
      moe::dered_indices_workspace_bytes(oep_size, num_experts, iep_size, num_local_experts);
  if (workspace == nullptr || !aligned(workspace, 4) || workspace_bytes < need)
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_dered_indices(tokens_per_expert_by_source, oep_size, num_experts,
                                              expert_start, iep_size, num_local_experts, capacity,
                                              indices, counts_by_dest, total, workspace, stream));
}

MOE_API moe_status_t moe_deredundency_combine_workspace_size(int64_t n, int64_t G,
                                                             size_t* bytes) {
  if (bytes == nullptr || n < 0 || n > INT32_MAX || G < 0 || G > INT32_MAX)
    return MOE_ERR_INVALID_ARG;
  *bytes = moe::dered_combine_workspace_bytes(n, G);
  return MOE_OK;
}

MOE_API moe_status_t moe_deredundency_combine(const void* outer_output, const float* router_coeff,
                                              const int32_t* dispatch_indices, int64_t n,
                                              int32_t H, int64_t G, void* whiteboard,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  if (n < 0 || n > INT32_MAX || G < 0 || G > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (moe_status_t s = check_h(H)) return s;
  if (n > 0 && (!row_ok(outer_output) || !word_ok(dispatch_indices))) return MOE_ERR_INVALID_ARG;
  if (router_coeff != nullptr && !aligned(router_coeff, 4)) return MOE_ERR_INVALID_ARG;
  if (G > 0 && !row_ok(whiteboard)) return MOE_ERR_INVALID_ARG;
  if (G > 0 && (workspace == nullptr || !aligned(workspace, 4) ||
                workspace_bytes < moe::dered_combine_workspace_bytes(n, G)))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_dered_combine(u16(outer_output), router_coeff, dispatch_indices, n,
                                              H, G, u16(whiteboard), workspace, stream));
}
