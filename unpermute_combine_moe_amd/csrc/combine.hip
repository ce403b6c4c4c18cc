// Weighted top-K unpermute-combine with zero / copy / constant experts and an
// unweighted shared-expert term.
//
// Follows the torch_npu.npu_moe_distribute_combine_v2 page, 计算公式 (output =
// sum of expert_scales * expert output + shared_expert_x; Moe(ori_x) = 0,
// ori_x and alpha_1*ori_x + alpha_2*v for the zero, copy and constant experts)
// and 参数说明 (the shared expert carries no weight), with the gather of the
// expert_parallel.py coverage page (_unpermute).
//
// One wave per token. Lane k gathers slot k's metadata (kind, row through the
// optional row map, probability, const index and coefficients) with vector
// loads; the values are broadcast to the wave with readlane. Each lane then
// walks 16-byte chunks of the hidden dim, issues the K row loads of a chunk
// back to back (non-temporal: every row is read once), accumulates them in
// fp32 in slot order, adds the shared row, rounds once to bf16 and stores.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;

enum SlotKind : int { kDrop = 0, kRow = 1, kCopy = 2, kConst = 3 };

// kAlphaPerH: the const-expert coefficients vary along h (stride_h != 0);
// otherwise they are one pair per (token, const expert), read with the slot
// metadata. kUnit: the permute backward -- every slot with a row has weight
// 1 and there are no ids, special experts or shared term.
// kMaxK: the slot arrays are sized for K <= kMaxK (8 or 16).
template <bool kHasRowMap, bool kAlphaPerH, bool kUnit, int kMaxK>
__global__ void __launch_bounds__(kWaves * kWave)
k_combine(const uint16_t* __restrict__ expert_out, int64_t N, const int32_t* __restrict__ row_of_slot,
          const int32_t* __restrict__ row_map, const int32_t* __restrict__ ids,
          const float* __restrict__ probs, SlotMask mk, int64_t T, int K, int H, int E,
          SpecialArgs sp, const uint16_t* __restrict__ shared_x, uint16_t* __restrict__ out,
          int nsplit) {
  // nsplit waves share a token, each taking every nsplit-th 64-chunk row of
  // the hidden dim (each writes its own part of the output row)
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int64_t t = uniform(static_cast<int>(blockIdx.x * (kWaves / nsplit) + w / nsplit));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  const int64_t copy_lo = int64_t(E) + sp.num_zero;
  const int64_t const_lo = copy_lo + sp.num_copy;
  const int64_t id_hi = const_lo + sp.num_const;

  // Slot metadata, lane k for slot k: one vector load per field (and one more
  // for the row map) instead of a chain of per-slot scalar loads.
  int m_kind = kDrop, m_src = 0;
  float m_p = 0.f, m_a1 = 0.f, m_a2 = 0.f;
  if (kUnit && lane < K) {
    const int64_t row = row_of_slot[t * K + lane];
    if (row >= 0 && row < N) {
      m_kind = kRow;
      m_src = static_cast<int>(row);
      m_p = 1.0f;
    }
  } else if (lane < K) {
    const int64_t s = t * K + lane;
    const int id_in = ids[s];
    const int id = mk.active(s) ? id_in : -1;  // a slot outside the mask is dropped
    m_p = probs[s];
    if (id >= 0 && id < E) {
      int64_t row = row_of_slot[s];
      if (kHasRowMap && row >= 0 && row < N) row = row_map[row];
      if (row >= 0 && row < N) {
        m_kind = kRow;
        m_src = static_cast<int>(row);
      }
    } else if (id >= copy_lo && id < const_lo) {
      m_kind = kCopy;
    } else if (id >= const_lo && id < id_hi) {
      m_kind = kConst;
      m_src = static_cast<int>(id - const_lo);
      if (!kAlphaPerH) {
        const int64_t ai = t * sp.a_st + int64_t(m_src) * sp.a_sc;
        m_a1 = sp.alpha1[ai];
        m_a2 = sp.alpha2[ai];
      }
    }
  }
  int kind[kMaxK], src[kMaxK];
  float p[kMaxK], a1[kMaxK], a2[kMaxK];
  bool need_ori = false;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    kind[k] = k < K ? __builtin_amdgcn_readlane(m_kind, k) : kDrop;
    src[k] = __builtin_amdgcn_readlane(m_src, k);
    p[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_p), k));
    a1[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_a1), k));
    a2[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_a2), k));
    need_ori |= kind[k] == kCopy || kind[k] == kConst;
  }

  const int chunks = H / 8;
  const uint16_t* orow = need_ori ? sp.ori_x + t * H : nullptr;
  for (int c = lane + part * kWave; c < chunks; c += kWave * nsplit) {
    const int h0 = c * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // loads of the routed rows first, so they are all in flight together
    Vec8 v[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (kind[k] == kRow) v[k] = load16_nt(expert_out + int64_t(src[k]) * H + h0);
    float o[8];
    if (need_ori) unpack8(load16(orow + h0), o);
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (kind[k] == kRow) {
        float f[8];
        unpack8(v[k], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(p[k], f[i], acc[i]);
      } else if (kind[k] == kCopy) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(p[k], o[i], acc[i]);
      } else if (kind[k] == kConst) {
        float cv[8];
        unpack8(load16(sp.const_v + int64_t(src[k]) * H + h0), cv);
        if (kAlphaPerH) {
          const int64_t abase = t * sp.a_st + int64_t(src[k]) * sp.a_sc;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int64_t ai = abase + int64_t(h0 + i) * sp.a_sh;
            const float val = sp.alpha1[ai] * o[i] + sp.alpha2[ai] * cv[i];
            acc[i] = __builtin_fmaf(p[k], val, acc[i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float val = a1[k] * o[i] + a2[k] * cv[i];
            acc[i] = __builtin_fmaf(p[k], val, acc[i]);
          }
        }
      }
    }
    if (shared_x != nullptr) {
      float f[8];
      unpack8(load16_nt(shared_x + t * H + h0), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    store16_nt(out + t * H + h0, pack8(acc));
  }
}

// Two waves per token when there are too few tokens to give every SIMD
// several rounds of waves and each row has at least two 64-chunk rows.
// Waves per token: below kSplitBelowTokens a batch gives too few waves to keep
// every SIMD busy for several rounds, so long rows are shared by 4 waves (or 2).
int split_for(int64_t T, int H) {
  if (T >= kSplitBelowTokens) return 1;
  if (H / 8 >= 4 * kWave) return 4;
  return H / 8 >= 2 * kWave ? 2 : 1;
}

}  // namespace

hipError_t launch_combine(const uint16_t* expert_out, int64_t N, const int32_t* row_of_slot,
                          const int32_t* row_map, const int32_t* ids, const float* probs,
                          SlotMask mk, int64_t T, int K, int H, int E, const SpecialArgs& sp,
                          const uint16_t* shared_x, uint16_t* out, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const int nsplit = split_for(T, H);
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWaves / nsplit)));
  const dim3 block(kWaves * kWave);
  const bool per_h = sp.num_const > 0 && sp.a_sh != 0;
#define MOE_COMBINE_K(RM, PH, MK)                                                              \
  hipLaunchKernelGGL((k_combine<RM, PH, false, MK>), grid, block, 0, st, expert_out, N,       \
                     row_of_slot, row_map, ids, probs, mk, T, K, H, E, sp, shared_x, out, nsplit)
#define MOE_COMBINE(RM, PH) \
  {                                 \
    if (K <= 8)                     \
      MOE_COMBINE_K(RM, PH, 8);     \
    else                            \
      MOE_COMBINE_K(RM, PH, 16);    \
  }
  if (row_map != nullptr) {
    if (per_h) MOE_COMBINE(true, true) else MOE_COMBINE(true, false)
  } else {
    if (per_h) MOE_COMBINE(false, true) else MOE_COMBINE(false, false)
  }
#undef MOE_COMBINE
#undef MOE_COMBINE_K
  return hipGetLastError();
}

hipError_t launch_permute_grad(const uint16_t* d_permuted, int64_t N, const int32_t* row_of_slot,
                               int64_t T, int K, int H, uint16_t* d_x, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const int nsplit = split_for(T, H);
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWaves / nsplit)));
  const dim3 block(kWaves * kWave);
  if (K <= 8)
    hipLaunchKernelGGL((k_combine<false, false, true, 8>), grid, block, 0, st, d_permuted, N,
                       row_of_slot, nullptr, nullptr, nullptr, SlotMask{nullptr, 0, K}, T, K, H,
                       0, SpecialArgs{}, nullptr, d_x, nsplit);
  else
    hipLaunchKernelGGL((k_combine<false, false, true, 16>), grid, block, 0, st, d_permuted, N,
                       row_of_slot, nullptr, nullptr, nullptr, SlotMask{nullptr, 0, K}, T, K, H,
                       0, SpecialArgs{}, nullptr, d_x, nsplit);
  return hipGetLastError();
}

}  // namespace moe
