// Internal launchers behind the C ABI. Arguments are already validated by the
// API layer; every launcher only enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// x_active_mask: which slots take part in the exchange. m == nullptr: all of
// them; per_slot: one flag per slot [T*K], else one per token [T]. A slot
// that takes no part is treated as a dropped slot (no row, no term).
struct SlotMask {
  const uint8_t* m;
  int per_slot;
  int K;
  __device__ __forceinline__ bool active(int64_t s) const {
    if (m == nullptr) return true;
    const uint32_t i = per_slot ? static_cast<uint32_t>(s)
                                : static_cast<uint32_t>(s) / static_cast<uint32_t>(K);
    return m[i] != 0;
  }
};

size_t permute_workspace_bytes(int64_t T, int K, int E);
hipError_t launch_permute(const uint16_t* x, const int32_t* ids, SlotMask mk, int64_t T, int H,
                          int K, int E,
                          uint16_t* permuted, int32_t* sorted_slot, int32_t* row_of_slot,
                          int32_t* counts, int32_t* offsets, void* ws, hipStream_t st);

hipError_t launch_permute_rows(const uint16_t* x, const int32_t* row_of_slot, int64_t T, int H,
                               int K, int64_t N, uint16_t* permuted, hipStream_t st);

size_t reorder_workspace_bytes(int R, int E_local);
hipError_t launch_reorder(const uint16_t* x, const int32_t* counts, int R, int E_local, int64_t N,
                          int H, uint16_t* y, int32_t* perm, int32_t* inv_perm,
                          int32_t* tokens_per_expert, int32_t* offsets, void* ws, hipStream_t st);

struct SpecialArgs {
  int num_zero, num_copy, num_const;
  const uint16_t* ori_x;
  const float* alpha1;
  const float* alpha2;
  int64_t a_st, a_sc, a_sh;
  const uint16_t* const_v;
};

hipError_t launch_combine(const uint16_t* expert_out, int64_t N, const int32_t* row_of_slot,
                          const int32_t* row_map, const int32_t* ids, const float* probs,
                          SlotMask mk, int64_t T, int K, int H, int E, const SpecialArgs& sp,
                          const uint16_t* shared_x, uint16_t* out, hipStream_t st);

// Outputs of the combine backward (every pointer but d_probs nullable).
struct CombineGradArgs {
  uint16_t* d_expert_out;
  float* d_probs;
  uint16_t* d_ori_x;
  float* d_alpha1;
  float* d_alpha2;
  uint16_t* d_const_v;
};

// How the const-expert coefficients are laid out, as far as their gradient
// is concerned: owned by one token ((t, c) scalars whose spans do not overlap
// between tokens), shared by all tokens along h ([c, H] rows), shared and
// constant along h, or anything else (no gradient kernel for it).
enum class AlphaLayout { kNone, kPerToken, kSharedAlongH, kSharedScalar, kOther };
AlphaLayout classify_alpha(const SpecialArgs& sp, int H);

size_t combine_grad_workspace_bytes(int64_t T, int H, int num_const);
hipError_t launch_combine_grad(const uint16_t* grad_out, const uint16_t* expert_out, int64_t N,
                               const int32_t* row_of_slot, const int32_t* row_map,
                               const int32_t* ids, const float* probs, SlotMask mk, int64_t T,
                               int K, int H, int E, const SpecialArgs& sp,
                               const CombineGradArgs& o, void* ws, hipStream_t st);

hipError_t launch_permute_grad(const uint16_t* d_permuted, int64_t N, const int32_t* row_of_slot,
                               int64_t T, int K, int H, uint16_t* d_x, hipStream_t st);

hipError_t launch_unpermute_grad(const uint16_t* grad_out, const uint16_t* permuted, int64_t N,
                                 const int32_t* row_of_slot, const float* probs, int64_t T, int K,
                                 int H, uint16_t* d_permuted, float* d_probs, hipStream_t st);

size_t dered_indices_workspace_bytes(int oep, int E, int iep, int El);
hipError_t launch_dered_indices(const int32_t* counts, int oep, int E, int expert_start, int iep,
                                int El, int64_t capacity, int32_t* indices,
                                int32_t* counts_by_dest, int32_t* total, void* ws,
                                hipStream_t st);
size_t dered_combine_workspace_bytes(int64_t n, int64_t G);
hipError_t launch_dered_combine(const uint16_t* src, const float* coeff, const int32_t* indices,
                                int64_t n, int H, int64_t G, uint16_t* wb, void* ws,
                                hipStream_t st);

// CUs of the current device rounded down to a multiple of 8 (one per XCD slot)
int persistent_grid();
size_t bgemm_sched_bytes(int E);
// also clears the 256-byte zero row `zeros`
hipError_t launch_bgemm_sched(const int32_t* offsets, int E, int64_t N_cap, int32_t* ws,
                              uint16_t* zeros, hipStream_t st);
hipError_t launch_bgemm_kgroup(const uint16_t* A, int64_t lda, int M, const uint16_t* B,
                               int64_t ldb, int N, const int32_t* ws, int E,
                               const uint16_t* zeros, uint16_t* C0, uint16_t* C1, int split,
                               int64_t ldc, hipStream_t st);
size_t gemm_grad_workspace_bytes(int E, int64_t N_cap, int H, int I);
hipError_t launch_grouped_gemm_swiglu_grad(const uint16_t* x, const int32_t* offsets, int E,
                                           int64_t N_cap, int H, int I, const uint16_t* wg,
                                           const uint16_t* wu, const uint16_t* wd,
                                           const uint16_t* h, const uint16_t* dy, uint16_t* dx,
                                           uint16_t* dwg, uint16_t* dwu, uint16_t* dwd,
                                           const float* preact, void* ws, hipStream_t st);

size_t gemm_workspace_bytes(int E, int64_t N_cap, int H, int I);
hipError_t launch_grouped_gemm_swiglu(const uint16_t* x, const int32_t* offsets, int E,
                                      int64_t N_cap, int H, int I, const uint16_t* wg,
                                      const uint16_t* wu, const uint16_t* wd, uint16_t* h,
                                      uint16_t* y, float* preact, void* ws, hipStream_t st);

}  // namespace moe
