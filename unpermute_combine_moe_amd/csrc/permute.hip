// Stable expert-major token permute (count -> scan -> stable scatter -> row copy).
//
// Follows the bucketing of the expert_parallel.py coverage page
// (_generate_permute_indices keeps the order inside a block, _permute gathers
// x[permuted_indices]) and the twinkle grouped-matmul PR (permute as x[idx]):
// slot s = t*K + k with a real id lands at
//     expert_offsets[id] + #{ s' < s : id(s') == id }.
//
// Layout of the work: the T*K slots are cut into chunks of kChunkWaves waves x
// 64 lanes x `iters` slots; wave w of a chunk owns a contiguous run of
// 64*iters slots, so "earlier wave" means "earlier slots". Counts are kept per
// (expert, chunk) in an expert-major table; its exclusive scan gives every
// chunk its first row inside every bucket. No global atomics: rank assignment
// is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kChunkWaves = 4;
constexpr int kChunkThreads = kChunkWaves * kWave;
constexpr int kScanThreads = 1024;

struct PermutePlan {
  int iters;    // slots per lane per chunk
  int64_t chunk;
  int64_t nblk; // number of chunks
};

PermutePlan plan_for(int64_t S) {
  PermutePlan p;
  // at least 8 slots per lane; at most 1024 chunks so the scan table stays small
  p.iters = static_cast<int>(std::max<int64_t>(8, ceil_div(S, int64_t(kChunkThreads) * 1024)));
  p.chunk = int64_t(kChunkThreads) * p.iters;
  p.nblk = ceil_div(S, p.chunk);
  return p;
}

// Lanes of this wave holding the same key (key < 2^nbits).
__device__ __forceinline__ uint64_t match_key(int key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Per-chunk histogram: blk_hist[e * nblk + b] = #slots of chunk b with id e.
__global__ void __launch_bounds__(kChunkThreads)
k_route_count(const int32_t* __restrict__ ids, int64_t S, int E, int iters, int64_t nblk,
              int32_t* __restrict__ blk_hist) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += kChunkThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t base = b * int64_t(kChunkThreads) * iters;
  for (int j = 0; j < iters; ++j) {
    const int64_t s = base + int64_t(j) * kChunkThreads + threadIdx.x;
    if (s < S) {
      const int id = ids[s];
      if (id >= 0 && id < E) atomicAdd(&cnt[id], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunkThreads) blk_hist[int64_t(e) * nblk + b] = cnt[e];
}

// Exclusive scan of the expert-major (expert, chunk) table, in place, by one
// workgroup; also writes the per-expert counts and offsets.
__global__ void __launch_bounds__(kScanThreads)
k_route_scan(int32_t* __restrict__ table, int E, int64_t nblk, int32_t* __restrict__ counts,
             int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kScanThreads];
  __shared__ int32_t total_s;
  const int64_t L = int64_t(E) * nblk;
  const int64_t seg = ceil_div(L, kScanThreads);
  const int64_t lo = std::min<int64_t>(L, threadIdx.x * seg);
  const int64_t hi = std::min<int64_t>(L, lo + seg);
  int32_t sum = 0;
  for (int64_t i = lo; i < hi; ++i) sum += table[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the 1024 partial sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - sum;  // exclusive
  if (threadIdx.x == kScanThreads - 1) total_s = part[threadIdx.x];
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t c = table[i];
    table[i] = run;
    run += c;
  }
  __syncthreads();
  const int32_t total = total_s;
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    if (nblk == 0) {
      offsets[e] = 0;
      counts[e] = 0;
    } else {
      const int32_t start = table[int64_t(e) * nblk];
      const int32_t end = (e + 1 < E) ? table[int64_t(e + 1) * nblk] : total;
      offsets[e] = start;
      counts[e] = end - start;
    }
  }
  if (threadIdx.x == 0) offsets[E] = total;
}

// Stable scatter of slot indices: row_of_slot[s] and sorted_slot[row].
__global__ void __launch_bounds__(kChunkThreads)
k_route_scatter(const int32_t* __restrict__ ids, int64_t S, int E, int iters, int64_t nblk,
                const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
                int32_t* __restrict__ sorted_slot, int32_t* __restrict__ row_of_slot) {
  extern __shared__ int32_t run[];  // [kChunkWaves][E]
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (int i = threadIdx.x; i < kChunkWaves * E; i += kChunkThreads) run[i] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t wbase = b * int64_t(kChunkThreads) * iters + int64_t(w) * kWave * iters;
  int32_t* my = run + w * E;
  // pass 1: per-wave counts
  for (int j = 0; j < iters; ++j) {
    const int64_t s = wbase + int64_t(j) * kWave + lane;
    if (s < S) {
      const int id = ids[s];
      if (id >= 0 && id < E) atomicAdd(&my[id], 1);
    }
  }
  __syncthreads();
  // first row of every (wave, expert): chunk base plus the counts of earlier waves
  for (int e = threadIdx.x; e < E; e += kChunkThreads) {
    int32_t r = blk_base[int64_t(e) * nblk + b];
#pragma unroll
    for (int ww = 0; ww < kChunkWaves; ++ww) {
      const int32_t c = run[ww * E + e];
      run[ww * E + e] = r;
      r += c;
    }
  }
  __syncthreads();
  // pass 2: each wave walks its slots in order; lanes with equal ids are ranked
  // by lane index, and the group's lowest lane advances the running row.
  const int nbits = 32 - __builtin_clz(static_cast<unsigned>(E));  // keys 0..E fit
  for (int j = 0; j < iters; ++j) {
    const int64_t s = wbase + int64_t(j) * kWave + lane;
    int id = (s < S) ? ids[s] : -1;
    const bool real = id >= 0 && id < E;
    const int key = real ? id : E;
    const uint64_t same = match_key(key, nbits);
    const int rank = rank_below(same);
    int32_t row = -1;
    if (real) row = my[id] + rank;
    if (real && rank == 0) my[id] += __popcll(same);
    if (s < S) {
      row_of_slot[s] = row;
      if (real) sorted_slot[row] = static_cast<int32_t>(s);
    }
  }
  // rows past N (no slot maps there) read -1
  const int32_t N = offsets[E];
  const int64_t r_lo = b * int64_t(kChunkThreads) * iters;
  const int64_t r_hi = std::min<int64_t>(S, r_lo + int64_t(kChunkThreads) * iters);
  for (int64_t r = r_lo + threadIdx.x; r < r_hi; r += kChunkThreads)
    if (r >= N) sorted_slot[r] = -1;
}

// Row copy, token-major: each wave reads its token's row once and writes it to
// the K rows the token's slots landed on (16-byte vectors, coalesced).
constexpr int kRowWaves = 4;
__global__ void __launch_bounds__(kRowWaves * kWave)
k_permute_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ row_of_slot,
               int64_t T, int H, int K, int64_t S, uint16_t* __restrict__ permuted) {
  const int64_t t = uniform(static_cast<int>(blockIdx.x * kRowWaves + threadIdx.x / kWave));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  int32_t rows[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rows[k] = (k < K) ? row_of_slot[t * K + k] : -1;
  const int chunks = H / 8;
  const uint16_t* src = x + t * H;
  for (int c = lane; c < chunks; c += kWave) {
    const Vec8 v = load16(src + c * 8);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && rows[k] >= 0 && rows[k] < S) store16(permuted + int64_t(rows[k]) * H + c * 8, v);
    }
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int K, int E) {
  const PermutePlan p = plan_for(T * K);
  return static_cast<size_t>(std::max<int64_t>(1, p.nblk) * E) * sizeof(int32_t);
}

hipError_t launch_permute(const uint16_t* x, const int32_t* ids, int64_t T, int H, int K, int E,
                          uint16_t* permuted, int32_t* sorted_slot, int32_t* row_of_slot,
                          int32_t* counts, int32_t* offsets, void* ws, hipStream_t st) {
  const int64_t S = T * K;
  const PermutePlan p = plan_for(S);
  int32_t* table = static_cast<int32_t*>(ws);
  if (p.nblk > 0) {
    hipLaunchKernelGGL(k_route_count, dim3(static_cast<unsigned>(p.nblk)), dim3(kChunkThreads),
                       E * sizeof(int32_t), st, ids, S, E, p.iters, p.nblk, table);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kScanThreads), 0, st, table, E, p.nblk, counts,
                     offsets);
  if (p.nblk > 0) {
    hipLaunchKernelGGL(k_route_scatter, dim3(static_cast<unsigned>(p.nblk)), dim3(kChunkThreads),
                       kChunkWaves * E * sizeof(int32_t), st, ids, S, E, p.iters, p.nblk, table,
                       offsets, sorted_slot, row_of_slot);
    if (permuted != nullptr) {
      hipLaunchKernelGGL(k_permute_rows, dim3(static_cast<unsigned>(ceil_div(T, kRowWaves))),
                         dim3(kRowWaves * kWave), 0, st, x, row_of_slot, T, H, K, S, permuted);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
