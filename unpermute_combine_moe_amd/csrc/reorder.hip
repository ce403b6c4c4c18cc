// Rank-major -> expert-major reorder of a receive buffer.
//
// Follows the expert_parallel.py coverage page, _generate_permute_indices and
// _permute: the buffer holds blocks (r, e) in r-major order; expert compute
// wants them in (e, r) order, order inside a block kept. perm[i] is the source
// row of destination row i.
//
// One workgroup builds the block tables (two exclusive scans over R*E_local
// entries; for at most 1024 blocks every row workgroup does it itself instead);
// the row kernel then gives each workgroup a run of destination
// rows: one thread per row finds its block by binary search over the
// destination block starts, and the four waves copy the rows as 16-byte
// vectors.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kSetupThreads = 1024;
constexpr int kRowsPerWg = 16;
constexpr int kRowThreads = 256;
constexpr int kCopyBatch = 8;  // 16-byte chunks per lane in flight in the row copy

// ws layout (int32): src_rm[B] | cnt_em[B] | src_em[B] | dst_em[B] | total[1]
__global__ void __launch_bounds__(kSetupThreads)
k_reorder_setup(const int32_t* __restrict__ counts, int R, int El, int32_t* __restrict__ ws,
                int32_t* __restrict__ tokens_per_expert, int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kSetupThreads];
  const int B = R * El;
  int32_t* src_rm = ws;
  int32_t* cnt_em = ws + B;
  int32_t* src_em = ws + 2 * B;
  int32_t* dst_em = ws + 3 * B;
  int32_t* total_p = ws + 4 * B;
  // block counts in (e, r) order, negative counts read as 0
  for (int i = threadIdx.x; i < B; i += kSetupThreads) {
    const int e = i / R, r = i % R;
    cnt_em[i] = std::max(counts[r * El + e], 0);
    src_rm[i] = std::max(counts[i], 0);
  }
  __syncthreads();
  // starts of the blocks in the rank-major source buffer
  block_exclusive_scan<kSetupThreads>(src_rm, src_rm, B, part);
  for (int i = threadIdx.x; i < B; i += kSetupThreads) {
    const int e = i / R, r = i % R;
    src_em[i] = src_rm[r * El + e];
  }
  // starts of the blocks in the expert-major destination buffer
  const int32_t total = block_exclusive_scan<kSetupThreads>(cnt_em, dst_em, B, part);
  for (int e = threadIdx.x; e < El; e += kSetupThreads) {
    const int32_t start = dst_em[e * R];
    const int32_t end = (e + 1 < El) ? dst_em[(e + 1) * R] : total;
    offsets[e] = start;
    tokens_per_expert[e] = end - start;
  }
  if (threadIdx.x == 0) {
    offsets[El] = total;
    *total_p = total;
  }
}

// kScanHere (at most kFusedBlocks blocks): no setup launch; every workgroup
// loads the block counts into LDS and runs the two scans itself (a few KB of
// L2 reads per workgroup instead of a launch), and workgroup 0 writes the
// per-expert counts and offsets.
constexpr int kFusedBlocks = 1024;
template <bool kScanHere>
__global__ void __launch_bounds__(kRowThreads)
k_reorder_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ counts, int R, int El,
               const int32_t* __restrict__ ws, int B, int64_t N, int H, uint16_t* __restrict__ y,
               int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
               int32_t* __restrict__ tokens_per_expert, int32_t* __restrict__ offsets) {
  __shared__ int32_t src_of[kRowsPerWg];
  __shared__ int32_t s_src[kScanHere ? kFusedBlocks : 1];  // rank-major block starts
  __shared__ int32_t s_dst[kScanHere ? kFusedBlocks : 1];  // expert-major block starts
  __shared__ int32_t s_part[kScanHere ? kRowThreads : 1];
  int64_t total;
  if (kScanHere) {
    // block counts (negative counts read as 0): s_src in (r, e) order, s_dst in (e, r) order
    for (int i = threadIdx.x; i < B; i += kRowThreads) {
      const int e = i / R, r = i % R;
      s_src[i] = std::max(counts[i], 0);
      s_dst[i] = std::max(counts[r * El + e], 0);
    }
    __syncthreads();
    block_exclusive_scan<kRowThreads>(s_src, s_src, B, s_part);
    total = block_exclusive_scan<kRowThreads>(s_dst, s_dst, B, s_part);
    if (blockIdx.x == 0) {
      for (int e = threadIdx.x; e < El; e += kRowThreads) {
        const int32_t start = s_dst[e * R];
        const int32_t end = (e + 1 < El) ? s_dst[(e + 1) * R] : static_cast<int32_t>(total);
        offsets[e] = start;
        tokens_per_expert[e] = end - start;
      }
      if (threadIdx.x == 0) offsets[El] = static_cast<int32_t>(total);
    }
  } else {
    total = ws[4 * B];
  }
  const int32_t* src_em = ws + 2 * B;
  const int32_t* dst_em = kScanHere ? s_dst : ws + 3 * B;
  const int64_t i0 = int64_t(blockIdx.x) * kRowsPerWg;
  if (threadIdx.x < kRowsPerWg) {
    const int64_t i = i0 + threadIdx.x;
    int32_t src = -1;
    if (i < N && i < total) {
      // last block whose destination start is <= i (empty blocks share the
      // start of the next block, so they are skipped)
      int lo = 0, hi = B;  // invariant: dst_em[lo] <= i < dst_em[hi] (dst_em[B] = +inf)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (dst_em[mid] <= i) lo = mid; else hi = mid;
      }
      // the source start of block (e, r) = lo: rank-major block r * El + e
      const int64_t sstart = kScanHere ? s_src[(lo % R) * El + lo / R] : src_em[lo];
      const int64_t s = sstart + (i - dst_em[lo]);
      src = (s >= 0 && s < N) ? static_cast<int32_t>(s) : -1;
    }
    if (i < N) {
      perm[i] = src;
      if (inv_perm != nullptr) {
        if (src >= 0) inv_perm[src] = static_cast<int32_t>(i);
        if (i >= total) inv_perm[i] = -1;  // source rows past the total are never used
      }
    }
    src_of[threadIdx.x] = src;
  }
  __syncthreads();
  if (y == nullptr) return;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int chunks = H / 8;
  constexpr int kRowsPerWave = kRowsPerWg / (kRowThreads / kWave);
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int r = w * kRowsPerWave + rr;
    const int64_t i = i0 + r;
    const int32_t src = src_of[r];
    if (i >= N || src < 0) continue;
    const uint16_t* s = x + int64_t(src) * H;
    uint16_t* d = y + i * H;
    // a batch of kCopyBatch chunks per lane: all loads issued, then all stores
    for (int c0 = lane; c0 < chunks; c0 += kWave * kCopyBatch) {
      Vec8 v[kCopyBatch];
#pragma unroll
      for (int b = 0; b < kCopyBatch; ++b) {
        const int c = c0 + b * kWave;
        if (c < chunks) v[b] = load16_nt(s + c * 8);
      }
#pragma unroll
      for (int b = 0; b < kCopyBatch; ++b) {
        const int c = c0 + b * kWave;
        if (c < chunks) store16_nt(d + c * 8, v[b]);
      }
    }
  }
}

}  // namespace

size_t reorder_workspace_bytes(int R, int E_local) {
  return (static_cast<size_t>(R) * E_local * 4 + 1) * sizeof(int32_t);
}

hipError_t launch_reorder(const uint16_t* x, const int32_t* counts, int R, int E_local, int64_t N,
                          int H, uint16_t* y, int32_t* perm, int32_t* inv_perm,
                          int32_t* tokens_per_expert, int32_t* offsets, void* ws, hipStream_t st) {
  int32_t* w = static_cast<int32_t*>(ws);
  const int B = R * E_local;
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kRowsPerWg)));
  if (N > 0 && B <= kFusedBlocks) {
    hipLaunchKernelGGL(k_reorder_rows<true>, grid, dim3(kRowThreads), 0, st, x, counts, R,
                       E_local, w, B, N, H, y, perm, inv_perm, tokens_per_expert, offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_reorder_setup, dim3(1), dim3(kSetupThreads), 0, st, counts, R, E_local, w,
                     tokens_per_expert, offsets);
  if (N > 0) {
    hipLaunchKernelGGL(k_reorder_rows<false>, grid, dim3(kRowThreads), 0, st, x, counts, R,
                       E_local, w, B, N, H, y, perm, inv_perm, tokens_per_expert, offsets);
  }
  return hipGetLastError();
}

}  // namespace moe
