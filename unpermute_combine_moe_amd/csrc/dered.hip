// Deredundency dispatch indices and the whiteboard combine, on one GPU.
//
// Follows the expert_parallel.py coverage page:
//  - _generate_deredundency_dispatch_indices: each source rank's routed buffer
//    is expert-major, the sources' buffers are concatenated (the gathered
//    buffer); the outer expert range [expert_start, expert_start +
//    iep_size*num_local) is selected and ordered [iep_dst, local_expert,
//    oep_source], order inside a block kept.
//  - _scale_by_router_coeff and _scatter_add_first_dim: the selected rows come
//    back scaled by their router coefficient and are added into a zero buffer
//    of the gathered shape at their dispatch index.
//
// Index math: one workgroup scans the flattened count table (the first
// gathered row of every (source, expert) block) and the selected blocks in
// destination order; the index kernel then gives every output position its
// block by binary search, as the reorder does.
// Whiteboard: the dispatch indices are distinct (a selection of gathered
// rows), so the scatter-add is inverted into a gather: inv[r] = j for
// indices[j] = r, and every whiteboard row is written exactly once -- the
// scaled source row, or zeros. No atomics, no separate zero fill of the rows.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kSetupThreads = 1024;
constexpr int kIndexThreads = 256;
constexpr int kRowWaves = 4;
constexpr int kWbBatch = 4;  // 16-byte chunks per lane loaded before their stores

// ws layout (int32): flat[oep*E] | blk_start[B] | blk_cnt[B] | blk_dst[B] | total[1]
__global__ void __launch_bounds__(kSetupThreads)
k_dered_setup(const int32_t* __restrict__ counts, int oep, int E, int expert_start, int iep,
              int El, int32_t* __restrict__ ws, int32_t* __restrict__ counts_by_dest) {
  __shared__ int32_t part[kSetupThreads];
  const int64_t F = int64_t(oep) * E;
  const int B = iep * El * oep;
  int32_t* flat = ws;
  int32_t* blk_start = ws + F;
  int32_t* blk_cnt = blk_start + B;
  int32_t* blk_dst = blk_cnt + B;
  int32_t* total_p = blk_dst + B;
  for (int64_t i = threadIdx.x; i < F; i += kSetupThreads) flat[i] = max(counts[i], 0);
  __syncthreads();
  // first gathered row of block (s, e): the exclusive prefix of the row-major
  // table (every row of the sources before s, then source s's earlier experts)
  block_exclusive_scan<kSetupThreads>(flat, flat, F, part);
  // selected blocks in (d, l, s) order
  for (int b = threadIdx.x; b < B; b += kSetupThreads) {
    const int s = b % oep;
    const int dl = b / oep;  // d * El + l
    const int64_t cell = int64_t(s) * E + expert_start + dl;
    blk_start[b] = flat[cell];
    blk_cnt[b] = max(counts[cell], 0);
  }
  __syncthreads();
  const int32_t total = block_exclusive_scan<kSetupThreads>(blk_cnt, blk_dst, B, part);
  for (int dl = threadIdx.x; dl < iep * El; dl += kSetupThreads) {
    int32_t sum = 0;
    for (int s = 0; s < oep; ++s) sum += blk_cnt[dl * oep + s];
    counts_by_dest[dl] = sum;
  }
  if (threadIdx.x == 0) *total_p = total;
}

__global__ void __launch_bounds__(kIndexThreads)
k_dered_index(const int32_t* __restrict__ ws, int64_t F, int B, int64_t capacity,
              int32_t* __restrict__ indices, int32_t* __restrict__ total_out) {
  const int32_t* blk_start = ws + F;
  const int32_t* blk_dst = blk_start + 2 * B;
  const int64_t total = blk_dst[B];
  const int64_t i = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (i == 0 && total_out != nullptr) *total_out = static_cast<int32_t>(total);
  if (i >= capacity) return;
  int32_t v = -1;
  if (i < total) {
    // last block whose destination start is <= i (empty blocks share the start
    // of the next block, so they are skipped)
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (blk_dst[mid] <= i) lo = mid; else hi = mid;
    }
    v = static_cast<int32_t>(blk_start[lo] + (i - blk_dst[lo]));
  }
  indices[i] = v;
}

__global__ void __launch_bounds__(kIndexThreads)
k_inv_fill(int32_t* __restrict__ inv, int64_t G) {
  const int64_t r = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (r < G) inv[r] = -1;
}

__global__ void __launch_bounds__(kIndexThreads)
k_inv_scatter(const int32_t* __restrict__ indices, int64_t n, int64_t G, int32_t* __restrict__ inv) {
  const int64_t j = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (j >= n) return;
  const int64_t r = indices[j];
  if (r >= 0 && r < G) inv[r] = static_cast<int32_t>(j);
}

// A whiteboard element is 0 + coeff * value, added into a zero buffer: an
// exactly zero product (a zero coefficient, or a value of either sign of
// zero) gives +0, while a nonzero product keeps its sign even where it rounds
// to zero.
__device__ __forceinline__ uint32_t plus_zero_halves(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  lo = lo == 0x8000u ? 0u : lo;
  hi = hi == 0x8000u ? 0u : hi;
  return lo | (hi << 16);
}

__device__ __forceinline__ uint32_t scaled_bf16(float p, float v) {
  return (p == 0.0f || v == 0.0f) ? 0u : mul_to_bf16_exact(p, v);
}

// One wave per whiteboard row: the scaled source row (correctly rounded
// product of the fp32 coefficient and the bf16 value) or zeros.
__global__ void __launch_bounds__(kRowWaves * kWave)
k_whiteboard_rows(const uint16_t* __restrict__ src, const float* __restrict__ coeff,
                  const int32_t* __restrict__ inv, int64_t G, int H, uint16_t* __restrict__ wb) {
  const int64_t r = uniform(static_cast<int>(blockIdx.x * kRowWaves + threadIdx.x / kWave));
  if (r >= G) return;
  const int lane = threadIdx.x % kWave;
  const int64_t j = inv[r];
  const int chunks = H / 8;
  uint16_t* dst = wb + r * H;
  if (j < 0) {
    const Vec8 z{{0u, 0u, 0u, 0u}};
    for (int c = lane; c < chunks; c += kWave) store16_nt(dst + c * 8, z);
    return;
  }
  const uint16_t* s = src + j * H;
  if (coeff == nullptr) {
    for (int c = lane; c < chunks; c += kWave) {
      Vec8 v = load16_nt(s + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) v.w[i] = plus_zero_halves(v.w[i]);
      store16_nt(dst + c * 8, v);
    }
    return;
  }
  const float p = coeff[j];
  // kWbBatch chunks per lane: all loads issued before their stores
  for (int c0 = lane; c0 < chunks; c0 += kWave * kWbBatch) {
    Vec8 v[kWbBatch];
#pragma unroll
    for (int b = 0; b < kWbBatch; ++b) {
      const int c = c0 + b * kWave;
      if (c < chunks) v[b] = load16_nt(s + c * 8);
    }
#pragma unroll
    for (int b = 0; b < kWbBatch; ++b) {
      const int c = c0 + b * kWave;
      if (c >= chunks) continue;
      float f[8];
      unpack8(v[b], f);
      Vec8 d;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d.w[i] = scaled_bf16(p, f[2 * i]) | (scaled_bf16(p, f[2 * i + 1]) << 16);
      store16_nt(dst + c * 8, d);
    }
  }
}

}  // namespace

size_t dered_indices_workspace_bytes(int oep, int E, int iep, int El) {
  return (static_cast<size_t>(oep) * E + 3 * static_cast<size_t>(iep) * El * oep + 1) *
         sizeof(int32_t);
}

hipError_t launch_dered_indices(const int32_t* counts, int oep, int E, int expert_start, int iep,
                                int El, int64_t capacity, int32_t* indices,
                                int32_t* counts_by_dest, int32_t* total, void* ws,
                                hipStream_t st) {
  int32_t* w = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_dered_setup, dim3(1), dim3(kSetupThreads), 0, st, counts, oep, E,
                     expert_start, iep, El, w, counts_by_dest);
  const int64_t n = capacity > 0 ? capacity : 1;  // one thread at least, for *total
  hipLaunchKernelGGL(k_dered_index, dim3(static_cast<unsigned>(ceil_div(n, kIndexThreads))),
                     dim3(kIndexThreads), 0, st, w, int64_t(oep) * E, iep * El * oep, capacity,
                     indices, total);
  return hipGetLastError();
}

size_t dered_combine_workspace_bytes(int64_t G) {
  return static_cast<size_t>(G > 0 ? G : 1) * sizeof(int32_t);
}

hipError_t launch_dered_combine(const uint16_t* src, const float* coeff, const int32_t* indices,
                                int64_t n, int H, int64_t G, uint16_t* wb, void* ws,
                                hipStream_t st) {
  if (G == 0) return hipGetLastError();
  int32_t* inv = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_inv_fill, dim3(static_cast<unsigned>(ceil_div(G, kIndexThreads))),
                     dim3(kIndexThreads), 0, st, inv, G);
  if (n > 0)
    hipLaunchKernelGGL(k_inv_scatter, dim3(static_cast<unsigned>(ceil_div(n, kIndexThreads))),
                       dim3(kIndexThreads), 0, st, indices, n, G, inv);
  hipLaunchKernelGGL(k_whiteboard_rows, dim3(static_cast<unsigned>(ceil_div(G, kRowWaves))),
                     dim3(kRowWaves * kWave), 0, st, src, coeff, inv, G, H, wb);
  return hipGetLastError();
}

}  // namespace moe
