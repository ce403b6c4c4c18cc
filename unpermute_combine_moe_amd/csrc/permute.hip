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
// (expert, chunk); a chunk's first row inside bucket e is the offset of e plus
// the counts of e in earlier chunks. The chunk size keeps the count table
// small, so every scatter workgroup derives these from the whole table itself
// (two launches before the row copy). No global atomics: rank assignment is
// deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kChunkWaves = 4;
constexpr int kChunkThreads = kChunkWaves * kWave;

struct PermutePlan {
  int iters;    // slots per lane per chunk
  int64_t chunk;
  int64_t nblk; // number of chunks
};

// Threads that share one expert's walk of the count table: a power of two,
// at most a wave, with threads-per-expert x E within the workgroup.
__host__ __device__ inline int walk_threads(int E) {
  int t = 1;
  while (t < kWave && 2 * t * E <= kChunkThreads) t *= 2;
  return t;
}

// Chunks are sized so the (chunk, expert) count table holds at most
// kTableMax entries (every scatter workgroup reads all of it), with at least
// 8 / walk_threads(E) (and at least 2) slots per lane: more, smaller chunks
// lengthen the table walk, which walk_threads(E) threads per expert share,
// and shorten the counting and the scatter.
constexpr int64_t kTableMax = 16384;

PermutePlan plan_for(int64_t S, int E) {
  PermutePlan p;
  const int64_t target = std::max<int64_t>(1, std::min<int64_t>(256, kTableMax / E));
  const int min_iters = std::max(2, 8 / walk_threads(E));
  p.iters = static_cast<int>(
      std::max<int64_t>(min_iters, ceil_div(S, int64_t(kChunkThreads) * target)));
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

// Ids are read in batches of kBatch per lane: the loads of a batch are
// independent, so a batch costs one memory latency instead of kBatch.
constexpr int kBatch = 8;

// Per-chunk histogram, chunk-major: hist[b * E + e] = #slots of chunk b with id e.
__global__ void __launch_bounds__(kChunkThreads)
k_route_count(const int32_t* __restrict__ ids, SlotMask mk, int64_t S, int E, int iters,
              int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += kChunkThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t base = b * int64_t(kChunkThreads) * iters;
  for (int j0 = 0; j0 < iters; j0 += kBatch) {
    int id[kBatch];
    bool act[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t s = base + int64_t(j0 + q) * kChunkThreads + threadIdx.x;
      const bool in = j0 + q < iters && s < S;
      id[q] = in ? ids[s] : -1;
      act[q] = in && mk.active(s);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (act[q] && id[q] >= 0 && id[q] < E) atomicAdd(&cnt[id[q]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunkThreads) hist[b * E + e] = cnt[e];
}

// Stable scatter of the slots of chunk b, given chunk_base(e) = the first row
// of bucket e that belongs to this chunk: writes row_of_slot[s] and
// sorted_slot[row], and -1 into sorted_slot rows [N, S) of the chunk's range.
template <typename ChunkBase>
__device__ void scatter_chunk(const int32_t* __restrict__ ids, SlotMask mk, int64_t S, int E,
                              int iters,
                              int64_t b, ChunkBase chunk_base, int32_t N, int32_t* run,
                              int32_t* __restrict__ sorted_slot, int32_t* __restrict__ row_of_slot) {
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (int i = threadIdx.x; i < kChunkWaves * E; i += kChunkThreads) run[i] = 0;
  __syncthreads();
  const int64_t wbase = b * int64_t(kChunkThreads) * iters + int64_t(w) * kWave * iters;
  int32_t* my = run + w * E;
  // ids of slots wbase + (j0 + q) * 64 + lane, q < kBatch
  // (slots outside the active mask read as id -1)
  auto load_batch = [&](int j0, int id[kBatch]) {
    bool act[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t s = wbase + int64_t(j0 + q) * kWave + lane;
      const bool in = j0 + q < iters && s < S;
      id[q] = in ? ids[s] : -1;
      act[q] = in && mk.active(s);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) id[q] = act[q] ? id[q] : -1;
  };
  // pass 1: per-wave counts
  for (int j0 = 0; j0 < iters; j0 += kBatch) {
    int id[kBatch];
    load_batch(j0, id);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (id[q] >= 0 && id[q] < E) atomicAdd(&my[id[q]], 1);
  }
  __syncthreads();
  // first row of every (wave, expert): chunk base plus the counts of earlier waves
  for (int e = threadIdx.x; e < E; e += kChunkThreads) {
    int32_t r = chunk_base(e);
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
  for (int j0 = 0; j0 < iters; j0 += kBatch) {
    int id[kBatch];
    load_batch(j0, id);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (j0 + q >= iters) break;
      const int64_t s = wbase + int64_t(j0 + q) * kWave + lane;
      const bool real = id[q] >= 0 && id[q] < E;
      const int key = real ? id[q] : E;
      const uint64_t same = match_key(key, nbits);
      const int rank = rank_below(same);
      int32_t row = -1;
      if (real) row = my[id[q]] + rank;
      if (real && rank == 0) my[id[q]] += __popcll(same);
      if (s < S) {
        row_of_slot[s] = row;
        if (real) sorted_slot[row] = static_cast<int32_t>(s);
      }
    }
  }
  // rows past N (no slot maps there) read -1
  const int64_t r_lo = b * int64_t(kChunkThreads) * iters;
  const int64_t r_hi = std::min<int64_t>(S, r_lo + int64_t(kChunkThreads) * iters);
  for (int64_t r = r_lo + threadIdx.x; r < r_hi; r += kChunkThreads)
    if (r >= N) sorted_slot[r] = -1;
}

// Scan and scatter in one launch: every workgroup sums the chunk-major count
// table itself (per expert: all chunks, and the chunks before its own), scans
// the expert totals in LDS, and chunk 0 publishes counts and offsets.
__global__ void __launch_bounds__(kChunkThreads)
k_route_scan_scatter(const int32_t* __restrict__ ids, SlotMask mk, int64_t S, int E, int iters,
                     int64_t nblk,
                     const int32_t* __restrict__ hist, int32_t* __restrict__ counts,
                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                     int32_t* __restrict__ row_of_slot) {
  extern __shared__ int32_t sm[];  // run[kChunkWaves * E] | before[E] | off[E] | part[kChunkThreads]
  int32_t* run = sm;
  int32_t* before = sm + kChunkWaves * E;
  int32_t* off = before + E;
  int32_t* part = off + E;
  const int64_t b = blockIdx.x;
  // tpe consecutive threads (an aligned group inside one wave) share expert
  // e's walk, each taking every tpe-th chunk; their sums meet by xor shuffles
  const int tpe = walk_threads(E);
  for (int g = threadIdx.x; g < E * tpe; g += kChunkThreads) {
    const int e = g / tpe, sub = g % tpe;
    int32_t tot = 0, pre = 0;
    for (int64_t b0 = sub; b0 < nblk; b0 += int64_t(kBatch) * tpe) {
      int32_t c[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int64_t bq = b0 + int64_t(q) * tpe;
        c[q] = (bq < nblk) ? hist[bq * E + e] : 0;
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        tot += c[q];
        pre += (b0 + int64_t(q) * tpe < b) ? c[q] : 0;
      }
    }
    for (int o = tpe / 2; o > 0; o >>= 1) {
      tot += __shfl_xor(tot, o, kWave);
      pre += __shfl_xor(pre, o, kWave);
    }
    if (sub == 0) {
      off[e] = tot;
      before[e] = pre;
    }
  }
  __syncthreads();
  // exclusive scan of the expert totals: each thread a contiguous run of experts
  const int per = (E + kChunkThreads - 1) / kChunkThreads;
  const int lo = std::min(E, static_cast<int>(threadIdx.x) * per);
  const int hi = std::min(E, lo + per);
  int32_t sum = 0;
  for (int e = lo; e < hi; ++e) sum += off[e];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int o = 1; o < kChunkThreads; o <<= 1) {
    const int32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t acc = part[threadIdx.x] - sum;
  const int32_t N = part[kChunkThreads - 1];
  for (int e = lo; e < hi; ++e) {
    const int32_t c = off[e];
    off[e] = acc;
    if (b == 0) {
      counts[e] = c;
      offsets[e] = acc;
    }
    acc += c;
  }
  if (b == 0 && threadIdx.x == 0) offsets[E] = N;
  __syncthreads();
  scatter_chunk(
      ids, mk, S, E, iters, b, [&](int e) { return off[e] + before[e]; }, N, run, sorted_slot,
      row_of_slot);
}

__global__ void __launch_bounds__(kChunkThreads)
k_route_empty(int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += kChunkThreads) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

// Row copy, token-major: each wave reads its token's row once and writes it to
// the K rows the token's slots landed on (16-byte vectors, coalesced).
constexpr int kRowWaves = 4;
constexpr int kRowBatch = 4;  // 16-byte chunks per lane loaded before their stores
__global__ void __launch_bounds__(kRowWaves * kWave)
k_permute_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ row_of_slot,
               int64_t T, int H, int K, int64_t S, uint16_t* __restrict__ permuted, int nsplit) {
  // nsplit waves share a token, each taking every nsplit-th 64-chunk row of it
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int64_t t = uniform(static_cast<int>(blockIdx.x * (kRowWaves / nsplit) + w / nsplit));
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  int32_t rows[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rows[k] = (k < K) ? row_of_slot[t * K + k] : -1;
  const int chunks = H / 8;
  const uint16_t* src = x + t * H;
  // kRowBatch chunks per lane: all loads issued before their stores
  const int step = kWave * nsplit;
  for (int c0 = lane + part * kWave; c0 < chunks; c0 += step * kRowBatch) {
    Vec8 v[kRowBatch];
#pragma unroll
    for (int b = 0; b < kRowBatch; ++b) {
      const int c = c0 + b * step;
      if (c < chunks) v[b] = load16_nt(src + c * 8);
    }
#pragma unroll
    for (int b = 0; b < kRowBatch; ++b) {
      const int c = c0 + b * step;
      if (c >= chunks) continue;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < K && rows[k] >= 0 && rows[k] < S)
          store16(permuted + int64_t(rows[k]) * H + c * 8, v[b]);
      }
    }
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int K, int E) {
  const PermutePlan p = plan_for(T * K, E);
  return static_cast<size_t>(std::max<int64_t>(1, p.nblk) * E) * sizeof(int32_t);
}

hipError_t launch_permute(const uint16_t* x, const int32_t* ids, SlotMask mk, int64_t T, int H,
                          int K, int E, uint16_t* permuted, int32_t* sorted_slot, int32_t* row_of_slot,
                          int32_t* counts, int32_t* offsets, void* ws, hipStream_t st) {
  const int64_t S = T * K;
  const PermutePlan p = plan_for(S, E);
  int32_t* table = static_cast<int32_t*>(ws);
  if (p.nblk == 0) {  // no slots: zero counts and offsets
    hipLaunchKernelGGL(k_route_empty, dim3(1), dim3(kChunkThreads), 0, st, E, counts, offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_route_count, dim3(static_cast<unsigned>(p.nblk)), dim3(kChunkThreads),
                     E * sizeof(int32_t), st, ids, mk, S, E, p.iters, table);
  const size_t lds = (size_t(kChunkWaves) * E + 2 * E + kChunkThreads) * sizeof(int32_t);
  hipLaunchKernelGGL(k_route_scan_scatter, dim3(static_cast<unsigned>(p.nblk)),
                     dim3(kChunkThreads), lds, st, ids, mk, S, E, p.iters, p.nblk, table, counts,
                     offsets, sorted_slot, row_of_slot);
  if (permuted != nullptr) {
    // two waves per token when there are too few tokens for several rounds of waves
    const int nsplit = (H / 8 >= 2 * kWave && T < kSplitBelowTokens) ? 2 : 1;
    hipLaunchKernelGGL(k_permute_rows,
                       dim3(static_cast<unsigned>(ceil_div(T, kRowWaves / nsplit))),
                       dim3(kRowWaves * kWave), 0, st, x, row_of_slot, T, H, K, S, permuted,
                       nsplit);
  }
  return hipGetLastError();
}

}  // namespace moe
