// Unpermute backward: d_permuted (prob-scaled gather of grad_out) and d_probs
// (per-slot dot product over the hidden dim).
//
// Follows the "[sync] PR-40312: Update moe token unpermute DTensor support"
// page, 主要改动: npu_moe_token_unpermute_grad_v2 returns the gradient of
// permuted_tokens, which stays sharded on the hidden dim (elementwise in h),
// and the gradient of probs, which is Partial() (a sum over h).
//
// One wave per token. The slots' rows and probabilities are read once (lane k
// for slot k, broadcast by readlane) and the token's grad_out row is kept in
// registers (kCpl 16-byte chunks per lane, packed bf16); the wave then streams
// the permuted rows slot by slot, writes p * g as correctly rounded bf16 and
// reduces each slot's fp32 dot product. (Loading slot k + 1's row during slot
// k was measured slower: the extra registers cost more occupancy than the
// overlap gains.)
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
                 uint16_t* __restrict__ d_permuted, float* __restrict__ d_probs, int nsplit) {
  // nsplit waves share a token: part q takes the 64-chunk rows q, q + nsplit, ...
  // of the hidden dim, and the per-slot partial dot products meet in LDS
  __shared__ float xch[kWaves][16];
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int64_t t = uniform(static_cast<int>(blockIdx.x * (kWaves / nsplit) + w / nsplit));
  const bool live = t < T;
  if (nsplit == 1 && !live) return;
  const int lane = threadIdx.x % kWave;
  const int chunks = live ? H / 8 : 0;
  // this lane's chunk j of the row: 64-chunk row j * nsplit + part
  auto chunk = [&](int j) { return lane + (j * nsplit + part) * kWave; };
  // slot metadata up front: lane k loads slot k, readlane broadcasts it
  int m_row = -1;
  float m_p = 0.f;
  if (live && lane < K) {
    const int64_t r = row_of_slot[t * K + lane];
    m_row = (r >= 0 && r < N) ? static_cast<int>(r) : -1;
    m_p = probs[t * K + lane];
  }
  int row[16];
  float p[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    row[k] = k < K ? __builtin_amdgcn_readlane(m_row, k) : -1;
    p[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_p), k));
  }
  // the token's grad_out row stays packed (bf16) in registers
  Vec8 g[kCpl];
#pragma unroll
  for (int j = 0; j < kCpl; ++j) {
    const int c = chunk(j);
    g[j] = c < chunks ? load16(grad_out + t * H + c * 8) : Vec8{{0u, 0u, 0u, 0u}};
  }
  float mine = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k >= K) break;
    float dot = 0.f;
    if (row[k] >= 0) {
      Vec8 v[kCpl];
#pragma unroll
      for (int j = 0; j < kCpl; ++j) {
        const int c = chunk(j);
        if (c < chunks) v[j] = load16_nt(permuted + int64_t(row[k]) * H + c * 8);
      }
      uint16_t* drow = d_permuted + int64_t(row[k]) * H;
#pragma unroll
      for (int j = 0; j < kCpl; ++j) {
        const int c = chunk(j);
        if (c < chunks) {
          float f[8], gf[8];
          unpack8(v[j], f);
          unpack8(g[j], gf);
          Vec8 d;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            d.w[i] = mul_to_bf16_exact(p[k], gf[2 * i]) |
                     (mul_to_bf16_exact(p[k], gf[2 * i + 1]) << 16);
            dot = __builtin_fmaf(gf[2 * i], f[2 * i], dot);
            dot = __builtin_fmaf(gf[2 * i + 1], f[2 * i + 1], dot);
          }
          store16(drow + c * 8, d);
        }
      }
      dot = wave_sum(dot);
    }
    if (lane == k) mine = dot;  // 0 for a slot without a row
  }
  if (nsplit > 1) {
    if (part != 0 && lane < K) xch[w][lane] = mine;
    __syncthreads();
    if (part != 0 || !live) return;
    if (lane < K)
      for (int q = 1; q < nsplit; ++q) mine += xch[w + q][lane];  // partners in part order
  }
  if (lane < K) d_probs[t * K + lane] = mine;
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
  // two waves per token for long rows below 2 * kSplitBelowTokens tokens: the
  // register-resident row halves, so occupancy doubles
  const int nsplit = (H / 8 >= 4 * kWave && T < 2 * kSplitBelowTokens) ? 2 : 1;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWaves / nsplit)));
  const dim3 block(kWaves * kWave);
  const int cpl = static_cast<int>(ceil_div(H / 8, kWave * nsplit));
#define MOE_GRAD_CASE(C)                                                                        \
  if (cpl <= C) {                                                                               \
    hipLaunchKernelGGL(k_unpermute_grad<C>, grid, block, 0, st, grad_out, permuted, N,          \
                       row_of_slot, probs, T, K, H, d_permuted, d_probs, nsplit);               \
    return hipGetLastError();                                                                   \
  }
  MOE_GRAD_CASE(1)
  MOE_GRAD_CASE(2)
  MOE_GRAD_CASE(4)
  MOE_GRAD_CASE(8)
  MOE_GRAD_CASE(16)
#undef MOE_GRAD_CASE
  hipLaunchKernelGGL(k_unpermute_grad_any, dim3(static_cast<unsigned>(ceil_div(T, kWaves))), block,
                     0, st, grad_out, permuted, N, row_of_slot,
                     probs, T, K, H, d_permuted, d_probs);
  return hipGetLastError();
}

}  // namespace moe
