// Unpermute backward: d_permuted (prob-scaled gather of grad_out) and d_probs
// (per-slot dot product over the hidden dim).
//
// Follows the "[sync] PR-40312: Update moe token unpermute DTensor support"
// page, 主要改动: npu_moe_token_unpermute_grad_v2 returns the gradient of
// permuted_tokens, which stays sharded on the hidden dim (elementwise in h),
// and the gradient of probs, which is Partial() (a sum over h).
//
// One wave per token. The token's grad_out row is loaded once into registers
// (kCpl 16-byte chunks per lane); for each slot the wave streams the permuted
// row in, writes p * g as correctly rounded bf16, and reduces the fp32 dot
// product across the wave.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;

template <int kCpl>
__global__ void __launch_bounds__(kWaves * kWave)
k_unpermute_grad(const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ permuted,
                 int64_t N, const int32_t* __restrict__ row_of_slot,
                 const float* __restrict__ probs, int64_t T, int K, int H,
                 uint16_t* __restrict__ d_permuted, float* __restrict__ d_probs) {
  const int64_t t = uniform(static_cast<int>(blockIdx.x * kWaves + threadIdx.x / kWave));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  const int chunks = H / 8;
  float g[kCpl][8];
#pragma unroll
  for (int j = 0; j < kCpl; ++j) {
    const int c = lane + j * kWave;
    if (c < chunks) unpack8(load16(grad_out + t * H + c * 8), g[j]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) g[j][i] = 0.f;
  }
  for (int k = 0; k < K; ++k) {
    const int64_t s = t * K + k;
    const int64_t row = row_of_slot[s];
    if (row < 0 || row >= N) {
      if (lane == 0) d_probs[s] = 0.f;
      continue;
    }
    const float p = probs[s];
    const uint16_t* prow = permuted + row * H;
    uint16_t* drow = d_permuted + row * H;
    Vec8 pv[kCpl];
#pragma unroll
    for (int j = 0; j < kCpl; ++j) {
      const int c = lane + j * kWave;
      if (c < chunks) pv[j] = load16_nt(prow + c * 8);
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < kCpl; ++j) {
      const int c = lane + j * kWave;
      if (c < chunks) {
        float f[8];
        unpack8(pv[j], f);
        Vec8 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d.w[i] = mul_to_bf16_exact(p, g[j][2 * i]) | (mul_to_bf16_exact(p, g[j][2 * i + 1]) << 16);
          dot = __builtin_fmaf(g[j][2 * i], f[2 * i], dot);
          dot = __builtin_fmaf(g[j][2 * i + 1], f[2 * i + 1], dot);
        }
        store16(drow + c * 8, d);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) d_probs[s] = dot;
  }
}

// Hidden sizes beyond kCpl = 16 (H > 8192): loop over chunks, re-reading the
// grad_out row from cache for every slot.
__global__ void __launch_bounds__(kWaves * kWave)
k_unpermute_grad_any(const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ permuted,
                     int64_t N, const int32_t* __restrict__ row_of_slot,
                     const float* __restrict__ probs, int64_t T, int K, int H,
                     uint16_t* __restrict__ d_permuted, float* __restrict__ d_probs) {
  const int64_t t = uniform(static_cast<int>(blockIdx.x * kWaves + threadIdx.x / kWave));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  const int chunks = H / 8;
  for (int k = 0; k < K; ++k) {
    const int64_t s = t * K + k;
    const int64_t row = row_of_slot[s];
    if (row < 0 || row >= N) {
      if (lane == 0) d_probs[s] = 0.f;
      continue;
    }
    const float p = probs[s];
    float dot = 0.f;
    for (int c = lane; c < chunks; c += kWave) {
      float gf[8], f[8];
      unpack8(load16(grad_out + t * H + c * 8), gf);
      unpack8(load16(permuted + row * H + c * 8), f);
      Vec8 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d.w[i] = mul_to_bf16_exact(p, gf[2 * i]) | (mul_to_bf16_exact(p, gf[2 * i + 1]) << 16);
        dot = __builtin_fmaf(gf[2 * i], f[2 * i], dot);
        dot = __builtin_fmaf(gf[2 * i + 1], f[2 * i + 1], dot);
      }
      store16(d_permuted + row * H + c * 8, d);
    }
    dot = wave_sum(dot);
    if (lane == 0) d_probs[s] = dot;
  }
}

}  // namespace

hipError_t launch_unpermute_grad(const uint16_t* grad_out, const uint16_t* permuted, int64_t N,
                                 const int32_t* row_of_slot, const float* probs, int64_t T, int K,
                                 int H, uint16_t* d_permuted, float* d_probs, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWaves)));
  const dim3 block(kWaves * kWave);
  const int cpl = static_cast<int>(ceil_div(H / 8, kWave));
#define MOE_GRAD_CASE(C)                                                                        \
  if (cpl <= C) {                                                                               \
    hipLaunchKernelGGL(k_unpermute_grad<C>, grid, block, 0, st, grad_out, permuted, N,          \
                       row_of_slot, probs, T, K, H, d_permuted, d_probs);                       \
    return hipGetLastError();                                                                   \
  }
  MOE_GRAD_CASE(1)
  MOE_GRAD_CASE(2)
  MOE_GRAD_CASE(4)
  MOE_GRAD_CASE(8)
  MOE_GRAD_CASE(16)
#undef MOE_GRAD_CASE
  hipLaunchKernelGGL(k_unpermute_grad_any, grid, block, 0, st, grad_out, permuted, N, row_of_slot,
                     probs, T, K, H, d_permuted, d_probs);
  return hipGetLastError();
}

}  // namespace moe
