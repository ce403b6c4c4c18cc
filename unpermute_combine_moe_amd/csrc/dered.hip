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
// destination order (for tables and block lists of at most 2,048 entries every
// index workgroup runs those scans itself instead); the index kernel then
// gives every output position its block by binary search, as the reorder does.
// Whiteboard: the scatter-add is turned into a segmented gather by destination
// row. Each row's sources are counted (integer atomics: the counts do not
// depend on the order), an exclusive scan of the counts gives each row its
// segment of a source list, and every source index is placed in its row's
// segment (the scan is one workgroup up to 16,384 rows, two kernels beyond).
// One wave per whiteboard row then writes the row once: zeros for no
// source, the correctly rounded scaled row for one source (the common case:
// the dispatch indices name distinct rows), and for several sources their
// scaled rows summed in fp32 in ascending source order (the order the
// page's scatter-add applies them), rounded once. No floating-point atomics,
// so the result does not depend on scheduling.
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

// kFused (count tables and block lists of at most kDeredFused entries): no
// setup launch; every workgroup runs the setup's two scans itself in LDS (an
// 8 KB L2 read of the counts per workgroup instead of a launch), and workgroup
// 0 writes the per-destination counts.
constexpr int kDeredFused = 2048;
template <bool kFused>
__global__ void __launch_bounds__(kIndexThreads)
k_dered_index(const int32_t* __restrict__ ws, int64_t F, int B, int64_t capacity,
              int32_t* __restrict__ indices, int32_t* __restrict__ total_out,
              const int32_t* __restrict__ counts, int oep, int E, int expert_start, int iep_el,
              int32_t* __restrict__ counts_by_dest) {
  __shared__ int32_t s_flat[kFused ? kDeredFused : 1];
  __shared__ int32_t s_start[kFused ? kDeredFused : 1];
  __shared__ int32_t s_cnt[kFused ? kDeredFused : 1];
  __shared__ int32_t s_dst[kFused ? kDeredFused : 1];
  __shared__ int32_t s_part[kFused ? kIndexThreads : 1];
  const int32_t* blk_start;
  const int32_t* blk_dst;
  int64_t total;
  if (kFused) {
    // the setup's scans, as k_dered_setup runs them
    for (int i = threadIdx.x; i < F; i += kIndexThreads) s_flat[i] = max(counts[i], 0);
    __syncthreads();
    block_exclusive_scan<kIndexThreads>(s_flat, s_flat, F, s_part);
    for (int b = threadIdx.x; b < B; b += kIndexThreads) {
      const int src = b % oep;
      const int dl = b / oep;
      const int64_t cell = int64_t(src) * E + expert_start + dl;
      s_start[b] = s_flat[cell];
      s_cnt[b] = max(counts[cell], 0);
    }
    __syncthreads();
    total = block_exclusive_scan<kIndexThreads>(s_cnt, s_dst, B, s_part);
    if (blockIdx.x == 0) {
      for (int dl = threadIdx.x; dl < iep_el; dl += kIndexThreads) {
        int32_t sum = 0;
        for (int src = 0; src < oep; ++src) sum += s_cnt[dl * oep + src];
        counts_by_dest[dl] = sum;
      }
    }
    blk_start = s_start;
    blk_dst = s_dst;
  } else {
    blk_start = ws + F;
    blk_dst = blk_start + 2 * B;
    total = blk_dst[B];
  }
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

// ---------------------------------------------------------------- whiteboard
// ws layout (int32): cnt[G] | start[G + 1] | one[G] | bsum[nb] | list[n],
// nb = ceil(G / kScanBlock); one[r] = the single source of row r, -1 for none,
// -2 for several (the row kernel's one-load path for the common case)
constexpr int kScanThreads = 256;
constexpr int kScanPer = 16;
constexpr int kScanBlock = kScanThreads * kScanPer;

__global__ void __launch_bounds__(kIndexThreads)
k_wb_clear(int32_t* __restrict__ cnt, int32_t* __restrict__ one, int64_t G) {
  const int64_t r = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (r < G) {
    cnt[r] = 0;
    one[r] = -1;
  }
}

__global__ void __launch_bounds__(kIndexThreads)
k_wb_count(const int32_t* __restrict__ indices, int64_t n, int64_t G, int32_t* __restrict__ cnt) {
  const int64_t j = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (j >= n) return;
  const int64_t r = indices[j];
  if (r >= 0 && r < G) atomicAdd(&cnt[r], 1);
}

// Sum of each block of kScanBlock counts.
__global__ void __launch_bounds__(kScanThreads)
k_wb_block_sums(const int32_t* __restrict__ cnt, int64_t G, int32_t* __restrict__ bsum) {
  __shared__ int32_t part[kScanThreads];
  const int64_t base = int64_t(blockIdx.x) * kScanBlock + int64_t(threadIdx.x) * kScanPer;
  int32_t v = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) v += (base + i < G) ? cnt[base + i] : 0;
  part[threadIdx.x] = v;
  __syncthreads();
  for (int o = kScanThreads / 2; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = part[0];
}

// start[r] = exclusive prefix of cnt; start[G] = number of placed sources.
// cnt is cleared again, to count the placements. Each workgroup first adds up
// the sums of the blocks before its own (a few loads: G / 4096 blocks).
__global__ void __launch_bounds__(kScanThreads)
k_wb_block_scan(int32_t* __restrict__ cnt, int64_t G, const int32_t* __restrict__ bsum,
                int32_t* __restrict__ start) {
  __shared__ int32_t part[kScanThreads];
  int32_t earlier = 0;
  for (int64_t j = threadIdx.x; j < int64_t(blockIdx.x); j += kScanThreads) earlier += bsum[j];
  part[threadIdx.x] = earlier;
  __syncthreads();
  for (int o = kScanThreads / 2; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  const int32_t block_base = part[0];
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kScanBlock + int64_t(threadIdx.x) * kScanPer;
  int32_t v[kScanPer];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    v[i] = (base + i < G) ? cnt[base + i] : 0;
    sum += v[i];
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int32_t x = static_cast<int>(threadIdx.x) >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  int32_t run = block_base + part[threadIdx.x] - sum;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    if (base + i < G) {
      start[base + i] = run;
      cnt[base + i] = 0;
    }
    run += v[i];
    if (base + i == G - 1) start[G] = run;
  }
}

// The whole scan in one workgroup, for up to kOneScanMax rows. Each of the 16
// waves owns a contiguous segment of the counts and reads it 64 at a time
// (one coalesced row per step, kept in registers); the wave totals are
// scanned in LDS, then each wave walks its rows again in order, carrying the
// running prefix with a wave-level inclusive scan per row. start[r] is the
// exclusive prefix, start[G] the total; cnt is cleared for the placement.
constexpr int kOneWaves = 16;
constexpr int kOneRows = 64;   // 64-element rows per wave
constexpr int kOneBatch = 16;  // rows loaded together
// Past 16,384 rows the scan over blocks of kScanBlock counts (two launches) is
// faster (at 65,536 rows: 125.6 against 141.2 us for the whole combine, when
// it still took three launches).
constexpr int64_t kOneScanMax = 16384;
static_assert(kOneScanMax <= int64_t(kOneWaves) * kOneRows * kWave, "one workgroup's capacity");
__global__ void __launch_bounds__(kOneWaves * kWave)
k_wb_scan_one(int32_t* __restrict__ cnt, int64_t G64, int32_t* __restrict__ start) {
  __shared__ int32_t wsum[kOneWaves];
  const int G = static_cast<int>(G64);  // <= kOneScanMax
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int rows = static_cast<int>(ceil_div(G, kOneWaves * kWave));  // rows per wave
  const int b0 = w * rows * kWave;
  int32_t tot = 0;
  for (int i0 = 0; i0 < rows; i0 += kOneBatch) {
    int32_t v[kOneBatch];
#pragma unroll
    for (int i = 0; i < kOneBatch; ++i) {
      const int r = b0 + (i0 + i) * kWave + lane;
      v[i] = (i0 + i < rows && r < G) ? cnt[r] : 0;
    }
#pragma unroll
    for (int i = 0; i < kOneBatch; ++i) tot += v[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, kWave);
  if (lane == 0) wsum[w] = tot;
  __syncthreads();
  int32_t carry = 0;
  for (int ww = 0; ww < w; ++ww) carry += wsum[ww];
  for (int i0 = 0; i0 < rows; i0 += kOneBatch) {
    int32_t v[kOneBatch];
#pragma unroll
    for (int i = 0; i < kOneBatch; ++i) {
      const int r = b0 + (i0 + i) * kWave + lane;
      v[i] = (i0 + i < rows && r < G) ? cnt[r] : 0;
    }
#pragma unroll
    for (int i = 0; i < kOneBatch; ++i) {
      if (i0 + i >= rows) break;
      const int r = b0 + (i0 + i) * kWave + lane;
      int32_t incl = v[i];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int32_t x = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += x;
      }
      if (r < G) {
        start[r] = carry + incl - v[i];
        cnt[r] = 0;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
  }
  if (w == kOneWaves - 1 && lane == 0) start[G] = carry;
}

// Every source index into its row's segment (order inside a segment is
// arbitrary here; the row kernel reads a segment in ascending source order).
__global__ void __launch_bounds__(kIndexThreads)
k_wb_place(const int32_t* __restrict__ indices, int64_t n, int64_t G,
           const int32_t* __restrict__ start, int32_t* __restrict__ fill,
           int32_t* __restrict__ list, int32_t* __restrict__ one) {
  const int64_t j = int64_t(blockIdx.x) * kIndexThreads + threadIdx.x;
  if (j >= n) return;
  const int64_t r = indices[j];
  if (r < 0 || r >= G) return;
  const int32_t s0 = start[r];
  list[s0 + atomicAdd(&fill[r], 1)] = static_cast<int32_t>(j);
  // every source of a row with several writes the same -2
  one[r] = (start[r + 1] - s0 == 1) ? static_cast<int32_t>(j) : -2;
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

// One source: the scaled row (correctly rounded product of the fp32
// coefficient and the bf16 value), or the row itself without coefficients.
__device__ void wb_single_row(const uint16_t* __restrict__ s, const float* __restrict__ coeff,
                              int64_t j, int chunks, int lane, uint16_t* __restrict__ dst) {
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

// The q-th smallest source index of a segment of L > 1 entries. Up to 64
// entries sit one per lane (rank by comparison with every other lane); longer
// segments are walked by repeatedly taking the smallest index above the
// previous one (indices in a segment are distinct).
__device__ int32_t wb_nth(const int32_t* __restrict__ seg, int L, int q, int32_t prev, int lane,
                          int32_t mine, int rank) {
  if (L <= kWave) {
    const uint64_t hit = ballot(lane < L && rank == q);
    return __shfl(mine, static_cast<int>(__builtin_ctzll(hit)), kWave);
  }
  int32_t best = INT32_MAX;
  for (int i = lane; i < L; i += kWave) {
    const int32_t v = seg[i];
    if (v > prev && v < best) best = v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = std::min(best, __shfl_xor(best, o, kWave));
  return best;
}

// One wave per whiteboard row.
constexpr int kWbSumChunks = 4;  // 16-byte chunks per lane accumulated per pass
__global__ void __launch_bounds__(kRowWaves * kWave)
k_whiteboard_rows(const uint16_t* __restrict__ src, const float* __restrict__ coeff,
                  const int32_t* __restrict__ start, const int32_t* __restrict__ list,
                  const int32_t* __restrict__ one, int64_t G, int H, uint16_t* __restrict__ wb) {
  const int64_t r = uniform(static_cast<int>(blockIdx.x * kRowWaves + threadIdx.x / kWave));
  if (r >= G) return;
  const int lane = threadIdx.x % kWave;
  const int32_t j1 = uniform(one[r]);
  const int chunks = H / 8;
  uint16_t* dst = wb + r * H;
  if (j1 == -1) {
    const Vec8 z{{0u, 0u, 0u, 0u}};
    for (int c = lane; c < chunks; c += kWave) store16_nt(dst + c * 8, z);
    return;
  }
  if (j1 >= 0) {
    wb_single_row(src + int64_t(j1) * H, coeff, j1, chunks, lane, dst);
    return;
  }
  const int32_t s0 = uniform(start[r]);
  const int L = uniform(start[r + 1] - s0);
  const int32_t* seg = list + s0;
  // several sources: ranks of the first 64 entries (used when L <= 64)
  const int32_t mine = lane < L ? seg[lane] : INT32_MAX;
  int rank = 0;
  for (int i = 0; i < std::min(L, kWave); ++i) rank += (__shfl(mine, i, kWave) < mine) ? 1 : 0;
  for (int c0 = 0; c0 < chunks; c0 += kWave * kWbSumChunks) {
    float acc[kWbSumChunks][8];
#pragma unroll
    for (int b = 0; b < kWbSumChunks; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[b][i] = 0.f;
    int32_t prev = -1;
    for (int q = 0; q < L; ++q) {
      const int32_t j = wb_nth(seg, L, q, prev, lane, mine, rank);
      prev = j;
      const float p = coeff ? coeff[j] : 1.0f;
      const uint16_t* s = src + int64_t(j) * H;
#pragma unroll
      for (int b = 0; b < kWbSumChunks; ++b) {
        const int c = c0 + b * kWave + lane;
        if (c >= chunks) continue;
        float f[8];
        unpack8(load16(s + c * 8), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b][i] = __builtin_fmaf(p, f[i], acc[b][i]);
      }
    }
#pragma unroll
    for (int b = 0; b < kWbSumChunks; ++b) {
      const int c = c0 + b * kWave + lane;
      if (c < chunks) store16_nt(dst + c * 8, pack8(acc[b]));
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
  const int64_t F = int64_t(oep) * E;
  const int B = iep * El * oep;
  const int64_t n = capacity > 0 ? capacity : 1;  // one thread at least, for *total
  const dim3 grid(static_cast<unsigned>(ceil_div(n, kIndexThreads)));
  if (F <= kDeredFused && B <= kDeredFused) {
    hipLaunchKernelGGL(k_dered_index<true>, grid, dim3(kIndexThreads), 0, st, w, F, B, capacity,
                       indices, total, counts, oep, E, expert_start, iep * El, counts_by_dest);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_dered_setup, dim3(1), dim3(kSetupThreads), 0, st, counts, oep, E,
                     expert_start, iep, El, w, counts_by_dest);
  hipLaunchKernelGGL(k_dered_index<false>, grid, dim3(kIndexThreads), 0, st, w, F, B, capacity,
                     indices, total, counts, oep, E, expert_start, iep * El, counts_by_dest);
  return hipGetLastError();
}

size_t dered_combine_workspace_bytes(int64_t n, int64_t G) {
  const int64_t nb = ceil_div(G, kScanBlock);
  return static_cast<size_t>(G + (G + 1) + G + nb + n + 1) * sizeof(int32_t);
}

hipError_t launch_dered_combine(const uint16_t* src, const float* coeff, const int32_t* indices,
                                int64_t n, int H, int64_t G, uint16_t* wb, void* ws,
                                hipStream_t st) {
  if (G == 0) return hipGetLastError();
  const int64_t nb = ceil_div(G, kScanBlock);
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* start = cnt + G;
  int32_t* one = start + (G + 1);
  int32_t* bsum = one + G;
  int32_t* list = bsum + nb;
  const dim3 gG(static_cast<unsigned>(ceil_div(G, kIndexThreads)));
  hipLaunchKernelGGL(k_wb_clear, gG, dim3(kIndexThreads), 0, st, cnt, one, G);
  if (n > 0)
    hipLaunchKernelGGL(k_wb_count, dim3(static_cast<unsigned>(ceil_div(n, kIndexThreads))),
                       dim3(kIndexThreads), 0, st, indices, n, G, cnt);
  if (G <= kOneScanMax) {
    hipLaunchKernelGGL(k_wb_scan_one, dim3(1), dim3(kOneWaves * kWave), 0, st, cnt, G, start);
  } else {
    hipLaunchKernelGGL(k_wb_block_sums, dim3(static_cast<unsigned>(nb)), dim3(kScanThreads), 0,
                       st, cnt, G, bsum);
    hipLaunchKernelGGL(k_wb_block_scan, dim3(static_cast<unsigned>(nb)), dim3(kScanThreads), 0,
                       st, cnt, G, bsum, start);
  }
  if (n > 0)
    hipLaunchKernelGGL(k_wb_place, dim3(static_cast<unsigned>(ceil_div(n, kIndexThreads))),
                       dim3(kIndexThreads), 0, st, indices, n, G, start, cnt, list, one);
  hipLaunchKernelGGL(k_whiteboard_rows, dim3(static_cast<unsigned>(ceil_div(G, kRowWaves))),
                     dim3(kRowWaves * kWave), 0, st, src, coeff, start, list, one, G, H, wb);
  return hipGetLastError();
}

}  // namespace moe
