// Weight-gradient GEMMs of the SwiGLU expert FFN backward (gfx950 bf16 MFMA).
//
// Follows the twinkle grouped-matmul PR ("feat(moe): NPU平台 EP experts forward
// 计算改用 NPU grouped matmul"), differentiated: with dh = dy Wd^T and
// (dg, du) from the SwiGLU derivative,
//   dWd = h^T dy,  [dWg | dWu] = x^T [dg | du]   (sums over each expert's rows)
// (the row-grouped products dh and dx = [dg | du] [Wg ; Wu]^T run on the
// forward's grouped kernel, with B stored [n][k]).
//
// k_bgemm_kgroup: C_e = A_e^T B_e with A_e [rows of e][m] and B_e [rows of
// e][n] (both row-contiguous): the contraction runs over the expert's rows,
// its ragged tail is zero-filled, and an expert without rows gets a zero
// tile. Tiles go out biggest expert first. One 128 x 256 output tile per
// workgroup (256 threads as 2 x 2 waves, each 64 x 128 = 2 x 4 accumulators of
// v_mfma_f32_32x32x16_bf16, fp32); k-steps of 32 rows loaded straight into LDS
// (global_load_lds, no register staging and no LDS write instructions)
// through a three-stage ring. The tiles sit in LDS as [k][col] and the MFMA
// operand (8 consecutive k of one column per lane) is formed by
// ds_read_b64_tr_b16 transpose reads, as the forward kernel does for its
// weights.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

constexpr int TM = 128, TN = 256;
constexpr int kThreads = 256;
constexpr int kSchedThreads = 1024;
constexpr int kXcds = 8;
// k_bgemm_kgroup: k-step (rows of the contraction), direct-to-LDS loads per
// thread per operand and stage, operand tile and stage bytes, ring depth
constexpr int kKgTK = 32;
constexpr int kKgLoadsA = TM * kKgTK / 8 / kThreads;
constexpr int kKgLoadsB = TN * kKgTK / 8 / kThreads;
constexpr int kKgTileA = TM * kKgTK * 2;
constexpr int kKgStage = kKgTileA + TN * kKgTK * 2;
constexpr int kKgStages = 3;

// [k][col] tile: k row, 16-byte column chunk c (16 per row)
template <int W>
__device__ __forceinline__ int swz_kc(int k, int c) { return k * (W / 8) + (c ^ (4 * (k & 3))); }

// Byte offsets of the two transpose reads that form the operand of columns
// col0 .. col0 + 31 of a [k][col] tile at k-substep 0 (substep kk adds 16 k
// rows, which keeps k & 3 and so the swizzle): within each group of 16 lanes,
// input lane i points at k row i / 4 (+ 4 for the second read), column 4 (i % 4).
template <int W>
__device__ __forceinline__ void tr_offsets(int col0, int lane, int off[2]) {
  const int g16 = lane / 16, i16 = lane % 16;
  const int n = col0 + 16 * (g16 % 2) + 4 * (i16 % 4);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 8 * (g16 / 2) + i16 / 4 + 4 * half;
    off[half] = swz_kc<W>(k, n / 8) * 16 + (n % 8) * 2;
  }
}

template <int W>
__device__ __forceinline__ bf16x8_t read_kc(const lds_u8_t* t, const int off[2], int kk) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(t + off[0] + kk * 16 * (W * 2)));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(t + off[1] + kk * 16 * (W * 2)));
  bf16x8_t r;
  __builtin_memcpy(&r, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
  return r;
}

// Epilogue of one wave's 64 x 128 accumulator block, rows m0 .. m0 + 63 and
// columns n0 .. n0 + 127. In registers a lane holds row m0 + 32 i + lane % 32
// and four consecutive columns n0 + 32 j + 8 q + 4 (lane / 32), so a direct
// store would cover 32 rows x 16 B. The block goes through the wave's 16 KB
// staging area `stg` in LDS as [64 rows][256 B] of bf16 (16-byte chunks
// XOR-swizzled by row % 16, which keeps both the column-wise writes and the
// row-wise reads free of bank conflicts) and is read back 16 B (8 columns)
// per lane, 4 rows x 256 B per wave-wide access.
__device__ __forceinline__ void stage_block(const f32x16_t acc[2][4], lds_u8_t* stg, int lane) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * i + lane % 32;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2_t packed = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
        const int chunk = (4 * j + q) ^ (r & 15);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
            stg + r * 256 + chunk * 16 + (lane / 32) * 8) = packed;
      }
  }
  // the wave's own writes have completed before it reads them back
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Staged row r (0..63), 16-byte chunk c (columns 8 c .. 8 c + 7 of the block).
__device__ __forceinline__ u32x4_t staged_chunk(const lds_u8_t* stg, int r, int c) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
      stg + r * 256 + (c ^ (r & 15)) * 16);
}

// The block stored as bf16 (columns at or past `split` go to C1 at column
// n - split; rows >= m_end and columns >= n_end are not stored).
__device__ __forceinline__ void store_block(const f32x16_t acc[2][4], lds_u8_t* stg, int m0,
                                            int m_end, int n0, int n_end, int split,
                                            uint16_t* C0, uint16_t* C1, int64_t ldc, int lane) {
  stage_block(acc, stg, lane);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int r = 4 * t + lane / 16, c = lane % 16;
    const u32x4_t v = staged_chunk(stg, r, c);
    const int m = m0 + r, n = n0 + 8 * c;
    if (m < m_end && n < n_end) {
      uint16_t* dst = n < split ? C0 + int64_t(m) * ldc + n : C1 + int64_t(m) * ldc + (n - split);
      *reinterpret_cast<u32x4_t*>(dst) = v;
    }
  }
}

// ws layout (int32): prefix[E+1] | offs[E+1] | order[E]
//   prefix: row-tile prefix (ceil(rows_e / TM) per expert), offs: clamped
//   offsets, order: experts by row count, largest first (ties: lower id first).
// Also clears the 256-byte zero row that the contraction's ragged tail reads.
__global__ void __launch_bounds__(kSchedThreads)
k_bgemm_sched(const int32_t* __restrict__ offsets, int E, int64_t N_cap, int32_t* __restrict__ ws,
              uint32_t* __restrict__ zeros) {
  __shared__ int32_t part[kSchedThreads];
  if (threadIdx.x < 64) zeros[threadIdx.x] = 0u;
  __shared__ int32_t rows[kSchedThreads];
  int32_t* prefix = ws;
  int32_t* offs = ws + (E + 1);
  int32_t* order = ws + 2 * (E + 1);
  const int e = threadIdx.x;
  int32_t lo = 0, hi = 0;
  if (e < E) {
    lo = static_cast<int32_t>(std::min<int64_t>(std::max(offsets[e], 0), N_cap));
    hi = static_cast<int32_t>(std::min<int64_t>(std::max(offsets[e + 1], 0), N_cap));
    hi = std::max(hi, lo);
  }
  rows[e] = hi - lo;
  const int32_t tiles = (e < E) ? (hi - lo + TM - 1) / TM : 0;
  part[e] = tiles;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int32_t v = e >= off ? part[e - off] : 0;
    __syncthreads();
    part[e] += v;
    __syncthreads();
  }
  if (e < E) {
    prefix[e] = part[e] - tiles;
    offs[e] = lo;
    if (e == E - 1) {
      prefix[E] = part[e];
      offs[E] = hi;
    }
    int rank = 0;
    const int32_t mine = rows[e];
    for (int o = 0; o < E; ++o) rank += (rows[o] > mine || (rows[o] == mine && o < e)) ? 1 : 0;
    order[rank] = e;
  }
}

// k-grouped C_e = A_e^T B_e over the rows of expert e: A rows [row][m] (lda),
// B rows [row][n] (ldb); C_e is [M][N] at C0 + e * M * ldc (columns at or past
// `split` go to C1 + e * M * ldc at column n - split). Grid: E * m-tiles *
// n-tiles, experts taken in `order` (largest first). Its own k-step of kKgTK
// rows and a ring of kKgStages direct-to-LDS stages (16 KB each), so that three
// workgroups fit a CU: the tiles of small experts are short and latency-bound,
// and more of them in flight is what they need.
__global__ void __launch_bounds__(kThreads, 2)
k_bgemm_kgroup(const uint16_t* __restrict__ A, int64_t lda, int M, const uint16_t* __restrict__ B,
               int64_t ldb, int N, const int32_t* __restrict__ ws, int E,
               const uint16_t* __restrict__ zeros, uint16_t* __restrict__ C0,
               uint16_t* __restrict__ C1, int split, int64_t ldc, int bm, int bn) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kKgStages * kKgStage];
  lds_u8_t* lds = (lds_u8_t*)smem;
  const int32_t* offs = ws + (E + 1);
  const int32_t* order = ws + 2 * (E + 1);
  const int mt_n = (M + TM - 1) / TM, nt_n = (N + TN - 1) / TN;
  const int per_e = mt_n * nt_n;
  const int e = order[static_cast<int>(blockIdx.x) / per_e];
  const int t = static_cast<int>(blockIdx.x) % per_e;
  // Which output tile of expert e: with bm > 0 (per_e a multiple of 8), the
  // workgroups of XCD t % 8 take one bm x bn block of the (m, n) tile grid,
  // chosen on the host so that the A column blocks and B column blocks each
  // XCD reads (from its own L2) add up to the fewest bytes; else row-major.
  int mt, nt;
  if (bm > 0) {
    const int x = t % kXcds, i = t / kXcds;
    const int gn = nt_n / bn;  // XCD blocks along n
    mt = (x / gn) * bm + i / bn;
    nt = (x % gn) * bn + i % bn;
  } else {
    mt = t / nt_n;
    nt = t % nt_n;
  }
  const int m0 = mt * TM, n0 = nt * TN;
  const int r_lo = offs[e], r_hi = offs[e + 1];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;

  // Direct-to-LDS loads: load l fills slot c = l * 256 + wave * 64 + lane of
  // each [k][col] operand tile, i.e. k row c / (W / 8) and swizzled chunk
  // c % (W / 8) for a tile W columns wide (A: 128, B: 256), so the lane loads
  // global column chunk (c % (W / 8)) ^ 4 (k & 3).
  int krowA[kKgLoadsA], colA[kKgLoadsA], krowB[kKgLoadsB], colB[kKgLoadsB];
#pragma unroll
  for (int l = 0; l < kKgLoadsA; ++l) {
    const int c = l * kThreads + wave * kWave + lane;
    krowA[l] = c >> 4;
    const int cc = (c & 15) ^ (4 * (krowA[l] & 3));
    colA[l] = std::min(m0 + cc * 8, M - 8);
  }
#pragma unroll
  for (int l = 0; l < kKgLoadsB; ++l) {
    const int c = l * kThreads + wave * kWave + lane;
    krowB[l] = c >> 5;
    const int cc = (c & 31) ^ (4 * (krowB[l] & 3));
    colB[l] = std::min(n0 + cc * 8, N - 8);
  }
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int ksteps = static_cast<int>(ceil_div(r_hi - r_lo, kKgTK));
  int issued = 0;
  auto issue = [&]() {
    const uint32_t st = uniform(static_cast<int>(lds0 + (issued % kKgStages) * kKgStage +
                                                 wave * kWave * 16));
    const int r0 = r_lo + issued * kKgTK;
#pragma unroll
    for (int l = 0; l < kKgLoadsA; ++l) {
      const int r = r0 + krowA[l];
      const bool in = r < r_hi;
      load_lds16(in ? A + int64_t(r) * lda + colA[l] : zeros, st + l * kThreads * 16);
    }
#pragma unroll
    for (int l = 0; l < kKgLoadsB; ++l) {
      const int r = r0 + krowB[l];
      const bool in = r < r_hi;
      load_lds16(in ? B + int64_t(r) * ldb + colB[l] : zeros, st + kKgTileA + l * kThreads * 16);
    }
    ++issued;
  };
  int offA[2][2], offB[4][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) tr_offsets<TM>(wm * 64 + 32 * i, lane, offA[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) tr_offsets<TN>(wn * 128 + 32 * j, lane, offB[j]);
  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // Stage i goes to buffer i % kKgStages, kKgStages - 1 stages ahead of the
  // multiply; the waits count only this thread's loads of later stages.
  while (issued < kKgStages - 1 && issued < ksteps) issue();
  for (int ks = 0; ks < ksteps; ++ks) {
    static_assert(kKgStages == 3, "one later stage at most is in flight at a wait");
    if (issued - ks - 1 >= 1) wait_vmcnt<kKgLoadsA + kKgLoadsB>();
    else wait_vmcnt<0>();
    // every wave's part of stage ks is in LDS, and every wave is done reading
    // stage ks - 1 (its MFMAs consumed those reads), whose buffer the issue
    // below refills
    stage_barrier();
    if (issued < ksteps) issue();
    const lds_u8_t* ta = lds + (ks % kKgStages) * kKgStage;
    const lds_u8_t* tb = ta + kKgTileA;
#pragma unroll
    for (int kk = 0; kk < kKgTK / 16; ++kk) {
      bf16x8_t fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = read_kc<TM>(ta, offA[i], kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = read_kc<TN>(tb, offB[j], kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }
  // every wave is done reading the stages before the epilogue stages its output
  wait_lds_reads();
  stage_barrier();
  const int64_t ebase = int64_t(e) * M * ldc;
  // the LDS is free: every wave has passed the k-loop's last barrier (or, for
  // an expert without rows, never used it)
  static_assert(4 * 16384 <= kKgStages * kKgStage, "the staging areas fit the ring");
  store_block(acc, lds + wave * 16384, m0 + wm * 64, M, n0 + wn * 128, N, split, C0 + ebase,
              C1 + ebase, ldc, lane);
}

}  // namespace

size_t bgemm_sched_bytes(int E) {
  return ((static_cast<size_t>(3 * E + 2) * 4 + 255) / 256) * 256;
}

hipError_t launch_bgemm_sched(const int32_t* offsets, int E, int64_t N_cap, int32_t* ws,
                              uint16_t* zeros, hipStream_t st) {
  hipLaunchKernelGGL(k_bgemm_sched, dim3(1), dim3(kSchedThreads), 0, st, offsets, E, N_cap, ws,
                     reinterpret_cast<uint32_t*>(zeros));
  return hipGetLastError();
}

hipError_t launch_bgemm_kgroup(const uint16_t* A, int64_t lda, int M, const uint16_t* B,
                               int64_t ldb, int N, const int32_t* ws, int E,
                               const uint16_t* zeros, uint16_t* C0, uint16_t* C1, int split,
                               int64_t ldc, hipStream_t st) {
  const int mt_n = static_cast<int>(ceil_div(M, TM)), nt_n = static_cast<int>(ceil_div(N, TN));
  const int64_t grid = int64_t(E) * mt_n * nt_n;
  // the per-XCD tile block (bm x bn, bm | mt_n, bn | nt_n, bm bn = tiles / 8)
  // that minimizes the column blocks read per XCD: A's M columns are read by
  // nt_n / bn XCDs, B's N columns by mt_n / bm
  int bm = 0, bn = 0;
  if ((mt_n * nt_n) % kXcds == 0) {
    const int per = mt_n * nt_n / kXcds;
    int64_t best = -1;
    for (int a = 1; a <= mt_n; ++a) {
      if (mt_n % a != 0 || per % a != 0) continue;
      const int b = per / a;
      if (nt_n % b != 0) continue;
      const int64_t cost = int64_t(M) * (nt_n / b) + int64_t(N) * (mt_n / a);
      if (best < 0 || cost < best) { best = cost; bm = a; bn = b; }
    }
  }
  hipLaunchKernelGGL(k_bgemm_kgroup, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, A,
                     lda, M, B, ldb, N, ws, E, zeros, C0, C1, split, ldc, bm, bn);
  return hipGetLastError();
}

}  // namespace moe
