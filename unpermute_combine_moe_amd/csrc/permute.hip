// Stable expert-major token permute (count -> scan -> stable scatter -> row copy).
//
// Follows the bucketing of the expert_parallel.py coverage page
// (_generate_permute_indices keeps the order inside a block, _permute gathers
// x[permuted_indices]) and the twinkle grouped-matmul PR (permute as x[idx]):
// slot s = t*K + k with a real id lands at
//     expert_offsets[id] + #{ s' < s : id(s') == id }.
//
// Layout of the work: the T*K slots are cut into chunks of 4 (or 16) waves x
// 64 lanes x `iters` slots; wave w of a chunk owns a contiguous run of
// 64*iters slots, so "earlier wave" means "earlier slots". Three launches:
//  1. per chunk: its (chunk, expert) count table row and every slot's rank
//     among the chunk's slots with its id (a wave-level match);
//  2. one workgroup scans the table: expert counts and offsets, and for every
//     chunk its first row in each bucket (offsets[e] plus the counts of e in
//     earlier chunks); for tables of at most kFusedTable entries every
//     workgroup of launch 3 does this itself instead (two launches in all);
//  3. per token: each slot's row (that first row plus its rank in the chunk),
//     both index maps, and the row copy.
// No global atomics: rank assignment is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kChunkWaves = 4;
constexpr int kChunkThreads = kChunkWaves * kWave;
constexpr int kChunkWavesWide = 16;  // chunks of a table the row kernel scans itself
constexpr int kMaxExpertsPermute = 1024;
constexpr int kMaxTopK = 16;

struct PermutePlan {
  int waves;    // waves per chunk (one workgroup of the rank kernel)
  int iters;    // slots per lane per chunk
  int64_t chunk;
  int64_t nblk; // number of chunks
};

// Chunks are sized so the (chunk, expert) count table holds at most
// kTableMax entries (one workgroup scans it), with at least two slots per lane.
constexpr int64_t kTableMax = 16384;
// Tables of at most kFusedTable entries are scanned by every row workgroup
// itself (no scan launch).
constexpr int kFusedTable = 4096;

PermutePlan plan_with(int64_t S, int E, int waves, int64_t table_max) {
  PermutePlan p;
  p.waves = waves;
  const int64_t threads = int64_t(waves) * kWave;
  const int64_t target = std::max<int64_t>(1, std::min<int64_t>(256, table_max / E));
  p.iters = static_cast<int>(std::max<int64_t>(2, ceil_div(S, threads * target)));
  p.chunk = threads * p.iters;
  p.nblk = ceil_div(S, p.chunk);
  return p;
}

// Four waves per chunk; when that table is too big for the row kernel's own
// scan, chunks of sixteen waves instead if their table fits it (at E >= 64
// the same slots per lane, so as many waves rank them; E <= 512 keeps the rank
// kernel's per-wave counts within 32 KB of LDS).
PermutePlan plan_for(int64_t S, int E) {
  const PermutePlan p = plan_with(S, E, kChunkWaves, kTableMax);
  if (p.nblk * E <= kFusedTable || E > 512) return p;
  const PermutePlan q = plan_with(S, E, kChunkWavesWide, kFusedTable);
  return q.nblk * E <= kFusedTable ? q : p;
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

// Pass 1 over a chunk: its histogram, chunk-major (table[b * E + e] = #slots of
// chunk b with id e), and every slot's rank inside the chunk among the slots
// with its id, stored in row_of_slot (-1 for slots without a row); the row
// kernel turns it into the row. Wave w of the chunk owns a contiguous run of
// slots; lanes holding the same id are found with a ballot per id bit (a
// wave-level match), ranked with mbcnt, and the group's lowest lane advances
// the wave's running count in LDS -- deterministic, no global atomics.
template <int kW>
__global__ void __launch_bounds__(kW * kWave)
k_route_rank(const int32_t* __restrict__ ids, SlotMask mk, int64_t S, int E, int iters,
             int32_t* __restrict__ table, int32_t* __restrict__ row_of_slot) {
  constexpr int kThreads = kW * kWave;
  extern __shared__ int32_t run[];  // [kW * E]
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t b = blockIdx.x;
  for (int i = threadIdx.x; i < kW * E; i += kThreads) run[i] = 0;
  __syncthreads();
  const int64_t wbase = b * int64_t(kThreads) * iters + int64_t(w) * kWave * iters;
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
  // per-wave counts (the first batch of ids is kept for the ranking pass,
  // which then needs no second load when a lane has at most kBatch slots)
  int id0[kBatch];
  load_batch(0, id0);
#pragma unroll
  for (int q = 0; q < kBatch; ++q)
    if (id0[q] >= 0 && id0[q] < E) atomicAdd(&my[id0[q]], 1);
  for (int j0 = kBatch; j0 < iters; j0 += kBatch) {
    int id[kBatch];
    load_batch(j0, id);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (id[q] >= 0 && id[q] < E) atomicAdd(&my[id[q]], 1);
  }
  __syncthreads();
  // the chunk's histogram, and the first rank of every (wave, expert) inside
  // the chunk: the counts of the earlier waves
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int32_t r = 0;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) {
      const int32_t c = run[ww * E + e];
      run[ww * E + e] = r;
      r += c;
    }
    table[b * E + e] = r;
  }
  __syncthreads();
  // each wave walks its slots in order
  const int nbits = 32 - __builtin_clz(static_cast<unsigned>(E));  // keys 0..E fit
  for (int j0 = 0; j0 < iters; j0 += kBatch) {
    int id[kBatch];
    if (j0 == 0) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) id[q] = id0[q];
    } else {
      load_batch(j0, id);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (j0 + q >= iters) break;
      const int64_t s = wbase + int64_t(j0 + q) * kWave + lane;
      const bool real = id[q] >= 0 && id[q] < E;
      const int key = real ? id[q] : E;
      const uint64_t same = match_key(key, nbits);
      const int rank = rank_below(same);
      int32_t local = -1;
      if (real) local = my[id[q]] + rank;
      if (real && rank == 0) my[id[q]] += __popcll(same);
      if (s < S) row_of_slot[s] = local;
    }
  }
}

// Pass 2, one workgroup: per expert, the exclusive prefix of its column of the
// count table (the rows of that expert in earlier chunks), the expert totals
// and their exclusive scan (counts, offsets); the table is overwritten with
// every chunk's first row per expert, offsets[e] + the earlier chunks' rows.
constexpr int kScanThreads = 1024;
__host__ __device__ inline int scan_threads_per_expert(int E) {
  int t = 1;
  while (t < kWave && 2 * t * E <= kScanThreads) t *= 2;
  return t;
}

// A column range of one thread holds at most this many chunks: nblk <=
// kTableMax / E chunks are shared by t = scan_threads_per_expert(E) threads with
// t * E > 512 (the loop stops at the first t with 2 t E > 1024), or t = 64 for
// E <= 8 (at most 256 chunks).
constexpr int kScanRange = 32;

__global__ void __launch_bounds__(kScanThreads)
k_route_scan(int E, int64_t nblk, int32_t* __restrict__ table, int32_t* __restrict__ counts,
             int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kMaxExpertsPermute];
  // tpe consecutive threads (an aligned group inside one wave) share expert
  // e's column, thread sub taking the contiguous chunk range [lo, hi), all of
  // whose entries it loads at once and keeps for the write-back
  const int tpe = scan_threads_per_expert(E);
  const int len = static_cast<int>(ceil_div(nblk, tpe));
  const int g = threadIdx.x;
  const int e = g / tpe, sub = g % tpe;
  const bool mine = e < E;
  // table indices fit 32 bits: nblk * E <= kTableMax
  const int lo = static_cast<int>(std::min<int64_t>(nblk, int64_t(sub) * len));
  const int hi = static_cast<int>(std::min<int64_t>(nblk, int64_t(lo) + len));
  int32_t c[kScanRange];
#pragma unroll
  for (int q = 0; q < kScanRange; ++q) c[q] = (mine && lo + q < hi) ? table[(lo + q) * E + e] : 0;
  int32_t sum = 0;
#pragma unroll
  for (int q = 0; q < kScanRange; ++q) sum += c[q];
  // inclusive prefix of the range sums inside the group, and the expert total
  int32_t incl = sum;
  for (int o = 1; o < tpe; o <<= 1) {
    const int32_t v = __shfl_up(incl, o, kWave);
    if (sub >= o) incl += v;
  }
  const int32_t total = __shfl(incl, (threadIdx.x % kWave) | (tpe - 1), kWave);
  if (mine && sub == 0) tot[e] = total;
  __syncthreads();
  // exclusive scan of the expert totals by the first wave: each lane a run of
  // ceil(E / 64) experts, then a wave prefix of the run sums
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (E + kWave - 1) / kWave;
    const int elo = std::min(E, lane * per), ehi = std::min(E, elo + per);
    int32_t run = 0;
    for (int x = elo; x < ehi; ++x) run += tot[x];
    int32_t pre = run;
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t v = __shfl_up(pre, o, kWave);
      if (lane >= o) pre += v;
    }
    int32_t acc = pre - run;
    for (int x = elo; x < ehi; ++x) {
      const int32_t cx = tot[x];
      counts[x] = cx;
      offsets[x] = acc;
      tot[x] = acc;  // now the expert's first row
      acc += cx;
    }
    if (lane == kWave - 1) offsets[E] = pre;
  }
  __syncthreads();
  // every chunk's first row per expert
  if (mine) {
    int32_t r = tot[e] + incl - sum;
#pragma unroll
    for (int q = 0; q < kScanRange; ++q) {
      if (lo + q < hi) table[(lo + q) * E + e] = r;
      r += c[q];
    }
  }
}

__global__ void __launch_bounds__(kChunkThreads)
k_route_empty(int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += kChunkThreads) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

// Pass 3, token-major: the rows of a token's slots (the chunk's first row for
// the slot's expert plus the slot's rank inside the chunk), both index maps,
// -1 for the rows past N, and the row copy: each wave reads its token's row
// once and writes it to the K rows its slots landed on (16-byte vectors,
// coalesced). The slots of the workgroup's tokens are resolved first, one
// thread each, and their rows shared through LDS.
//
// kScanHere (small tables, nblk * E <= kFusedTable): pass 2 is folded in. The
// table still holds the chunks' raw counts; every workgroup loads it into LDS
// and scans it itself (expert totals, their exclusive scan, and for each of
// its slots the counts of the slot's expert in earlier chunks), which costs a
// few KB of L2 reads per workgroup instead of a launch; workgroup 0 writes the
// counts and offsets.
constexpr int kRowWaves = 4;
constexpr int kRowBatch = 4;  // 16-byte chunks per lane loaded before their stores
constexpr int kTableLoads = kFusedTable / (kRowWaves * kWave);  // per thread
template <bool kScanHere>
__global__ void __launch_bounds__(kRowWaves * kWave)
k_permute_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, SlotMask mk,
               int64_t T, int H, int K, int E, int64_t chunk, int nblk,
               const int32_t* __restrict__ table, int32_t* __restrict__ counts,
               int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot,
               int32_t* __restrict__ sorted_slot, uint16_t* __restrict__ permuted, int nsplit) {
  __shared__ int32_t s_rows[kRowWaves * kMaxTopK];
  __shared__ int32_t s_tab[kScanHere ? kFusedTable : 1];
  __shared__ int32_t s_off[kScanHere ? kMaxExpertsPermute + 1 : 1];
  const int tokens = kRowWaves / nsplit;  // tokens of this workgroup
  const int64_t t0 = int64_t(blockIdx.x) * tokens;
  const int64_t S = T * K;
  // this wave's token and its share of the row; the first batch of the row's
  // loads goes out before the slots are resolved (it does not depend on them)
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int lt = w / nsplit;
  const int64_t t = t0 + lt;
  const int lane = threadIdx.x % kWave;
  const int chunks = H / 8;
  const uint16_t* src = x + t * H;
  const int step = kWave * nsplit;
  const bool copy = permuted != nullptr && t < T;
  Vec8 v0[kRowBatch];
  if (copy) {
#pragma unroll
    for (int bb = 0; bb < kRowBatch; ++bb) {
      const int c = lane + part * kWave + bb * step;
      if (c < chunks) v0[bb] = load16_nt(src + c * 8);
    }
  }
  int32_t N;
  if (kScanHere) {
    // the raw count table into LDS (all loads of a thread in flight together)
    const int n = nblk * E;
    int32_t v[kTableLoads];
#pragma unroll
    for (int q = 0; q < kTableLoads; ++q) {
      const int i = q * kRowWaves * kWave + threadIdx.x;
      v[q] = i < n ? table[i] : 0;
    }
#pragma unroll
    for (int q = 0; q < kTableLoads; ++q) {
      const int i = q * kRowWaves * kWave + threadIdx.x;
      if (i < n) s_tab[i] = v[q];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRowWaves * kWave) {
      int32_t sum = 0;
      for (int c = 0; c < nblk; ++c) sum += s_tab[c * E + e];
      s_off[e] = sum;
    }
    __syncthreads();
    // exclusive scan of the expert totals by the first wave: a run of
    // ceil(E / 64) experts per lane, then a wave prefix of the run sums
    if (threadIdx.x < kWave) {
      const int ln = threadIdx.x;
      const int per = (E + kWave - 1) / kWave;
      const int elo = std::min(E, ln * per), ehi = std::min(E, elo + per);
      int32_t run = 0;
      for (int e = elo; e < ehi; ++e) run += s_off[e];
      int32_t pre = run;
      for (int o = 1; o < kWave; o <<= 1) {
        const int32_t u = __shfl_up(pre, o, kWave);
        if (ln >= o) pre += u;
      }
      int32_t acc = pre - run;
      for (int e = elo; e < ehi; ++e) {
        const int32_t ce = s_off[e];
        if (blockIdx.x == 0) {
          counts[e] = ce;
          offsets[e] = acc;
        }
        s_off[e] = acc;
        acc += ce;
      }
      if (ln == kWave - 1) {
        s_off[E] = pre;
        if (blockIdx.x == 0) offsets[E] = pre;
      }
    }
    __syncthreads();
    N = s_off[E];
  } else {
    N = offsets[E];
  }
  // one thread per slot of the workgroup's tokens
  if (static_cast<int>(threadIdx.x) < tokens * K) {
    const int64_t s = t0 * K + threadIdx.x;
    int32_t row = -1;
    if (s < S) {
      const int32_t id = ids[s];
      const int32_t local = row_of_slot[s];
      if (local >= 0 && id >= 0 && id < E && mk.active(s)) {
        const int b = static_cast<int>(s / chunk);
        if (kScanHere) {
          int32_t first = s_off[id];  // the expert's first row, then its rows in earlier chunks
          for (int c = 0; c < b; ++c) first += s_tab[c * E + id];
          row = first + local;
        } else {
          row = table[b * E + id] + local;
        }
        sorted_slot[row] = static_cast<int32_t>(s);
      }
      row_of_slot[s] = row;
      if (s >= N) sorted_slot[s] = -1;  // rows past N (one slot per row)
    }
    s_rows[threadIdx.x] = row;
  }
  __syncthreads();
  if (!copy) return;
  // nsplit waves share a token, each taking every nsplit-th 64-chunk row of it
  int32_t rows[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) rows[k] = (k < K) ? s_rows[lt * K + k] : -1;
  // kRowBatch chunks per lane: all loads issued before their stores
  for (int c0 = lane + part * kWave; c0 < chunks; c0 += step * kRowBatch) {
    Vec8 v[kRowBatch];
    if (c0 == lane + part * kWave) {
#pragma unroll
      for (int bb = 0; bb < kRowBatch; ++bb) v[bb] = v0[bb];
    } else {
#pragma unroll
      for (int bb = 0; bb < kRowBatch; ++bb) {
        const int c = c0 + bb * step;
        if (c < chunks) v[bb] = load16_nt(src + c * 8);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kRowBatch; ++bb) {
      const int c = c0 + bb * step;
      if (c >= chunks) continue;
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        if (k < K && rows[k] >= 0 && rows[k] < S)
          store16(permuted + int64_t(rows[k]) * H + c * 8, v[bb]);
      }
    }
  }
}

// A routing already resolved (row_of_slot) applied to a token tensor, token-major:
// each wave reads its token's row once and writes it to the rows of its slots.
__global__ void __launch_bounds__(kRowWaves * kWave)
k_apply_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ row_of_slot, int64_t T,
             int H, int K, int64_t N, uint16_t* __restrict__ permuted, int nsplit) {
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int64_t t = int64_t(blockIdx.x) * (kRowWaves / nsplit) + w / nsplit;
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  int32_t rows[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) rows[k] = (k < K) ? row_of_slot[t * K + k] : -1;
  const int chunks = H / 8;
  const uint16_t* src = x + t * H;
  const int step = kWave * nsplit;
  for (int c0 = lane + part * kWave; c0 < chunks; c0 += step * kRowBatch) {
    Vec8 v[kRowBatch];
#pragma unroll
    for (int bb = 0; bb < kRowBatch; ++bb) {
      const int c = c0 + bb * step;
      if (c < chunks) v[bb] = load16_nt(src + c * 8);
    }
#pragma unroll
    for (int bb = 0; bb < kRowBatch; ++bb) {
      const int c = c0 + bb * step;
      if (c >= chunks) continue;
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        if (k < K && rows[k] >= 0 && rows[k] < N)
          store16(permuted + int64_t(rows[k]) * H + c * 8, v[bb]);
      }
    }
  }
}

}  // namespace

hipError_t launch_permute_rows(const uint16_t* x, const int32_t* row_of_slot, int64_t T, int H,
                               int K, int64_t N, uint16_t* permuted, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const int nsplit = (H / 8 >= 2 * kWave && T < kSplitBelowTokens) ? 2 : 1;
  hipLaunchKernelGGL(k_apply_rows, dim3(static_cast<unsigned>(ceil_div(T, kRowWaves / nsplit))),
                     dim3(kRowWaves * kWave), 0, st, x, row_of_slot, T, H, K, N, permuted, nsplit);
  return hipGetLastError();
}

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
  if (p.waves == kChunkWavesWide)
    hipLaunchKernelGGL(k_route_rank<kChunkWavesWide>, dim3(static_cast<unsigned>(p.nblk)),
                       dim3(kChunkWavesWide * kWave), size_t(kChunkWavesWide) * E * sizeof(int32_t),
                       st, ids, mk, S, E, p.iters, table, row_of_slot);
  else
    hipLaunchKernelGGL(k_route_rank<kChunkWaves>, dim3(static_cast<unsigned>(p.nblk)),
                       dim3(kChunkThreads), size_t(kChunkWaves) * E * sizeof(int32_t), st, ids, mk,
                       S, E, p.iters, table, row_of_slot);
  // two waves per token when there are too few tokens for several rounds of waves
  const int nsplit = (permuted != nullptr && H / 8 >= 2 * kWave && T < kSplitBelowTokens) ? 2 : 1;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kRowWaves / nsplit)));
  const int nblk = static_cast<int>(p.nblk);  // nblk * E <= kTableMax
  if (p.nblk * E <= kFusedTable) {
    hipLaunchKernelGGL(k_permute_rows<true>, grid, dim3(kRowWaves * kWave), 0, st, x, ids, mk, T,
                       H, K, E, p.chunk, nblk, table, counts, offsets, row_of_slot, sorted_slot,
                       permuted, nsplit);
  } else {
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kScanThreads), 0, st, E, p.nblk, table, counts,
                       offsets);
    hipLaunchKernelGGL(k_permute_rows<false>, grid, dim3(kRowWaves * kWave), 0, st, x, ids, mk, T,
                       H, K, E, p.chunk, nblk, table, counts, offsets, row_of_slot, sorted_slot,
                       permuted, nsplit);
  }
  return hipGetLastError();
}

}  // namespace moe
