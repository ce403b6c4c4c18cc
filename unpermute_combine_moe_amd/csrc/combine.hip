// Weighted top-K unpermute-combine with zero / copy / constant experts and an
// unweighted shared-expert term.
//
// Follows the torch_npu.npu_moe_distribute_combine_v2 page, 计算公式 (output =
// sum of expert_scales * expert output + shared_expert_x; Moe(ori_x) = 0,
// ori_x and alpha_1*ori_x + alpha_2*v for the zero, copy and constant experts)
// and 参数说明 (the shared expert carries no weight), with the gather of the
// expert_parallel.py coverage page (_unpermute).
//
// One wave per token. The slot metadata of the token (kind, row, probability,
// const index) is read once into registers; then each lane walks 16-byte
// chunks of the hidden dim, issues the K row loads of a chunk back to back and
// accumulates them in fp32 in slot order, adds the shared row, rounds once
// to bf16 and stores.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;

enum SlotKind : int { kDrop = 0, kRow = 1, kCopy = 2, kConst = 3 };

template <bool kHasRowMap>
__global__ void __launch_bounds__(kWaves * kWave)
k_combine(const uint16_t* __restrict__ expert_out, int64_t N, const int32_t* __restrict__ row_of_slot,
          const int32_t* __restrict__ row_map, const int32_t* __restrict__ ids,
          const float* __restrict__ probs, int64_t T, int K, int H, int E, SpecialArgs sp,
          const uint16_t* __restrict__ shared_x, uint16_t* __restrict__ out) {
  const int64_t t = uniform(static_cast<int>(blockIdx.x * kWaves + threadIdx.x / kWave));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  const int64_t copy_lo = int64_t(E) + sp.num_zero;
  const int64_t const_lo = copy_lo + sp.num_copy;
  const int64_t id_hi = const_lo + sp.num_const;

  int kind[16];
  int64_t src[16];  // row offset (elements) for kRow, const index for kConst
  float p[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    kind[k] = kDrop;
    src[k] = 0;
    p[k] = 0.f;
    if (k < K) {
      const int64_t s = t * K + k;
      const int id = ids[s];
      p[k] = probs[s];
      if (id >= 0 && id < E) {
        int64_t row = row_of_slot[s];
        if (kHasRowMap && row >= 0 && row < N) row = row_map[row];
        if (row >= 0 && row < N) {
          kind[k] = kRow;
          src[k] = row * H;
        }
      } else if (id >= copy_lo && id < const_lo) {
        kind[k] = kCopy;
      } else if (id >= const_lo && id < id_hi) {
        kind[k] = kConst;
        src[k] = id - const_lo;
      }
    }
  }

  const int chunks = H / 8;
  const uint16_t* orow = sp.ori_x ? sp.ori_x + t * H : nullptr;
  for (int c = lane; c < chunks; c += kWave) {
    const int h0 = c * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // loads of the routed rows first, so they are all in flight together
    Vec8 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (kind[k] == kRow) v[k] = load16(expert_out + src[k] + h0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (kind[k] == kRow) {
        float f[8];
        unpack8(v[k], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(p[k], f[i], acc[i]);
      } else if (kind[k] == kCopy) {
        float f[8];
        unpack8(load16(orow + h0), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(p[k], f[i], acc[i]);
      } else if (kind[k] == kConst) {
        float o[8], cv[8];
        unpack8(load16(orow + h0), o);
        unpack8(load16(sp.const_v + src[k] * H + h0), cv);
        const int64_t abase = t * sp.a_st + src[k] * sp.a_sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t ai = abase + int64_t(h0 + i) * sp.a_sh;
          const float val = sp.alpha1[ai] * o[i] + sp.alpha2[ai] * cv[i];
          acc[i] = __builtin_fmaf(p[k], val, acc[i]);
        }
      }
    }
    if (shared_x != nullptr) {
      float f[8];
      unpack8(load16(shared_x + t * H + h0), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    store16(out + t * H + h0, pack8(acc));
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* expert_out, int64_t N, const int32_t* row_of_slot,
                          const int32_t* row_map, const int32_t* ids, const float* probs,
                          int64_t T, int K, int H, int E, const SpecialArgs& sp,
                          const uint16_t* shared_x, uint16_t* out, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWaves)));
  if (row_map != nullptr)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(kWaves * kWave), 0, st, expert_out, N,
                       row_of_slot, row_map, ids, probs, T, K, H, E, sp, shared_x, out);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(kWaves * kWave), 0, st, expert_out, N,
                       row_of_slot, row_map, ids, probs, T, K, H, E, sp, shared_x, out);
  return hipGetLastError();
}

}  // namespace moe
