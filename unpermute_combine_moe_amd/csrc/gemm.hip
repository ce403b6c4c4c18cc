// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Follows the twinkle grouped-matmul PR ("feat(moe): NPU平台 EP experts forward
// 计算改用 NPU grouped matmul"): every expert group of the expert-major buffer
// goes through one grouped matmul plus SwiGLU instead of a per-expert loop.
//   pass 1 (gate/up):  h = bf16( silu(x Wg[e]) * (x Wu[e]) )   fp32 accumulate
//   pass 2 (down):     y = bf16( h Wd[e] )                      fp32 accumulate
// The same kernel runs the backward's row-grouped products: the gate/up
// recompute with the SwiGLU derivative, dh = dy Wd[e]^T (optionally turned
// straight into [dg | du] with kept pre-activations) and dx = [dg | du]
// [Wg[e] ; Wu[e]]^T, whose B operands are stored [n][k].
//
// Work decomposition. A small scheduling kernel turns the device-side expert
// offsets into a row-tile prefix (ceil(rows_e / BM) tiles per expert, 0 for an
// empty expert). Each GEMM pass is one persistent launch; a workgroup walks
// logical tiles (row tile, column tile) inside the range owned by its XCD, so
// the tiles that share an expert's weight panel and an A row-block run on the
// same XCD and reuse its L2.
//
// Tile: BM = 128 rows x 256 B-columns x BK = 64, 256 threads as 2 x 2 waves;
// each wave owns 64 rows x 128 B-columns = 2 x 4 MFMA 32x32 accumulators. The
// MFMA is fed the weight fragment as its first operand, i.e. it computes the
// transposed tile, so that each lane ends up with four consecutive output
// columns of one token row (8-byte writes into the epilogue's LDS staging).
// Pass 1 packs 128 gate columns and the matching 128 up columns into the 256
// B-columns, so the SwiGLU epilogue finds g and u of an output element in the
// same lane and register.
//
// Data path: both operand tiles go from global memory straight into LDS
// (16 bytes per lane, no register staging: buffer_load_dwordx4 ... lds for the
// A rows, bounded by the tile's valid rows, global_load_lds_dwordx4 for the
// weights) through a
// three-stage ring, so two k-steps of loads are in flight while one is
// multiplied; one s_barrier per k-step, with explicit vmcnt waits. Every
// k-step but a workgroup's last two issues the loads of the step two ahead;
// those run as a loop of their own so the steady-state body has no per-load
// branch. A is kept
// [row][k] and read with ds_read_b128. Weights stored [k][n] (the forward's,
// and the recompute's) stay in that layout in LDS and the MFMA B operand (8
// consecutive k of one column per lane) is formed by two ds_read_b64_tr_b16
// transpose reads: within each group of 16 lanes, output lane 4a+b takes
// element b of input lanes a, a+4, a+8, a+12, so input lane i points at row
// k0 + i/4, column 4*(i%4). Weights stored [n][k] (the backward's dh and dx)
// are loaded and read like the A rows.
// Both tiles are stored in 16-byte chunks with an XOR swizzle of the chunk
// index ([row][k]: by (row / 2) & 7, [k][n]: by 4 * (k & 3)) that keeps the
// operand reads free of bank conflicts; the swizzle is applied by choosing
// which global chunk each lane loads, since a direct-to-LDS load writes lane L
// at base + 16 L.
//
// Epilogue: the output fragments are staged in LDS (in the ring stage that the
// tile's last k-step has just freed) and written back row-contiguous with
// 16-byte buffer stores, so each store covers whole 128-byte lines; stores of
// padding rows carry an offset past the tile's valid rows and are dropped by
// the buffer range check.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = 128;
constexpr int BN = 256;  // B-columns per tile
constexpr int BK = 64;
constexpr int kChunksA = BM * BK / 8;  // 16-byte chunks per stage
constexpr int kChunksB = BN * BK / 8;
constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;

// (the row term (row / 2) & 7 spreads any 16 consecutive rows of 128 bytes
// over all 16 bank groups of 16 bytes)
__device__ __forceinline__ int swz(int row, int kc) { return row * (BK / 8) + (kc ^ ((row >> 1) & 7)); }


typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

constexpr int kStages = 3;
constexpr int kStageBytes = (kChunksA + kChunksB) * 16;

// Waves of a workgroup: 2 (64-row halves) x kWavesN (B-column blocks). The
// gate/up passes and the backward's dh use 4 waves (one per SIMD, 64 x 128
// each); the down pass, whose tiles are only 8 k-steps long, uses 8 (two per
// SIMD, 64 x 64 each), measured faster there (217 against 227 us) and not for
// gate/up; the backward's plain row GEMM (dx) uses 8 as well.
template <int kMode>
struct Layout {
  static constexpr int kWavesN = (kMode == 1 || kMode == 3) ? 4 : 2;
  static constexpr int kThreads = 2 * kWavesN * kWave;
  static constexpr int kColFrags = BN / 32 / kWavesN;     // 32-column MFMA blocks per wave
  static constexpr int kLoadsA = kChunksA / kThreads;     // direct-to-LDS loads per thread per stage
  static constexpr int kLoadsB = kChunksB / kThreads;
  static constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
  static constexpr int kReads = 2 + 2 * kColFrags;        // LDS fragment reads per sub-step
  static constexpr int kMfmas = 2 * kColFrags;            // MFMAs per sub-step
};
// kPaired: the tile's 256 B-columns are 128 gate and the matching 128 up
// columns (gate/up passes); otherwise 256 plain output columns. kBkc: B_e is
// stored [n][k] (k contiguous, the backward's dh and dx), loaded and read like
// the A rows; otherwise [k][n], read with transpose reads.
template <int kMode>
struct Mode {
  static constexpr bool kPaired = kMode == 0 || kMode == 2;
  static constexpr bool kBkc = kMode == 3 || kMode == 4;
};
// Epilogue. Each 32-row fragment of a wave's output goes through LDS: the
// lanes write their MFMA results (one token row per lane, four consecutive
// columns per register group) as packed bf16, then read the fragment back
// row-contiguous, 16 bytes per lane, and store it so that one store covers
// whole rows (4 rows x 256 B or 8 rows x 128 B) instead of 32 rows x 16 B.
// kRowBytes: bytes of one staged row (the wave's output columns; mode 2 puts
// dg and du side by side); 16-byte chunks are XOR-swizzled by row so that
// both the column-wise writes and the row-wise reads are free of bank
// conflicts. kStores counts the vector-memory stores a wave issues per tile.
template <int kMode>
struct EpiloguePlan {
  static constexpr int kOutFrags =
      Mode<kMode>::kPaired ? Layout<kMode>::kColFrags / 2 : Layout<kMode>::kColFrags;
  static constexpr int kRowBytes = kOutFrags * 64 * (kMode == 2 ? 2 : 1);
  static constexpr int kChunks = kRowBytes / 16;        // per staged row
  static constexpr int kRowsPerStore = kWave / kChunks;  // rows one wave-wide store covers
  static constexpr int kStoresPerFrag = 32 / kRowsPerStore;
  // mode 4 writes dg and du for every staged chunk of dh
  static constexpr int kStores = (kMode == 4 ? 4 : 2) * kStoresPerFrag;
  static constexpr int kWaveBytes = 32 * kRowBytes;     // staged rows of one fragment
  // Mode 0's optional fp32 pre-activations: per fragment, the wave's 64 g
  // columns and then its 64 u columns go through the staging area as rows of
  // 256 B (4 rows per wave-wide store); kPreStores counts their stores per tile.
  static constexpr int kPreStoresPerFrag = (kMode == 0) ? 2 * (32 / 4) : 0;
  static constexpr int kPreStores = 2 * kPreStoresPerFrag;
  static constexpr int kWaveStride = (kMode == 0) ? 32 * 256 : kWaveBytes;  // per-wave area
};

template <int kRowBytes>
__device__ __forceinline__ int stage_chunk(int row, int chunk) {
  // rows of 256 B start on the same bank: key = row % 16; rows of 128 B
  // alternate between the two bank halves: key = (row / 2) % 8
  return kRowBytes == 256 ? (chunk ^ (row & 15)) : (chunk ^ ((row >> 1) & 7));
  static_assert(kRowBytes == 256 || kRowBytes == 128, "staged row sizes");
}

__device__ __forceinline__ int swz_b(int k, int c) { return k * (BN / 8) + (c ^ (4 * (k & 3))); }

__device__ __forceinline__ bf16x8_t lds_read_a(const lds_u8_t* base, int slot) {
  const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(base + slot * 16);
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Direct-to-LDS loads of the k-loop with the fewest instructions. The A rows
// take the k-step offset in the buffer's scalar offset (the lane offset stays
// the tile's); each B source pointer advances one k-step in place, and that
// add also covers the wait state m0 needs before an LDS-DMA load. (m0 is set
// with s_mov: an add into m0 would write SCC, and an SCC clobber lets the
// compiler move the MFMAs out of the issue order the k-loop pins.)
__device__ __forceinline__ void buffer_load_lds16_at(i32x4_t rsrc, uint32_t voffset,
                                                     uint32_t soffset, uint32_t lds_base,
                                                     int off) {
  // the descriptor words made wave-uniform again here (free when they already
  // are), so the "s" operand never lands in VGPRs whatever the caller's code
  i32x4_t r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = __builtin_amdgcn_readfirstlane(rsrc[w]);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base + off), "v"(voffset), "s"(r), "s"(soffset)
               : "memory", "m0");
}
__device__ __forceinline__ void global_load_lds16_step(const uint16_t*& p, uint64_t adv,
                                                       uint32_t lds_base, int off) {
  asm volatile("s_mov_b32 m0, %1\n\tv_lshl_add_u64 %0, %2, 0, %0\n\tglobal_load_lds_dwordx4 %0, off"
               : "+v"(p)
               : "s"(lds_base + off), "s"(adv)
               : "memory", "m0");
}

// kMode 0: gate/up + SwiGLU -> h.  kMode 1: down -> y.
// kMode 0 with preact != nullptr also stores g and u (fp32) as preact [N, 2 Ncols].
// kMode 2: gate/up recomputed for the backward; with dh = aux [N, Ncols], the
// epilogue writes C [N, 2 * Ncols] = [dg | du], dg = dh * u * s (1 + g (1 - s)),
// du = dh * g * s, s = 1 / (1 + exp(-g)) (the SwiGLU derivative).
// kMode 3: C = A B_e^T with B_e = [B0[e] | B1[e]] stored [n][k] (B0 holding
// k < ksplit, B1 the rest; dx of the backward, and dh without kept
// pre-activations). kMode 4: the dh GEMM (B_e = Wd[e] stored [n][k]) whose
// epilogue rounds dh to bf16 and forms C [N, 2 * Ncols] = [dg | du] from the
// kept pre-activations preact [N, 2 Ncols] (read only).
template <int kMode>
__global__ void __launch_bounds__(Layout<kMode>::kThreads, 1)
k_gemm(const uint16_t* __restrict__ A, int Kdim, const uint16_t* __restrict__ B0,
       const uint16_t* __restrict__ B1, int Ncols, const int32_t* __restrict__ offsets, int E,
       int64_t N_cap, uint16_t* __restrict__ C, const uint16_t* __restrict__ aux,
       float* __restrict__ preact, int ksplit) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  // row-tile prefix and clamped expert offsets, built once per workgroup in LDS
  // for the per-tile expert lookup
  __shared__ int32_t s_prefix[kMaxExperts + 1];
  __shared__ int32_t s_offs[kMaxExperts + 1];
  lds_u8_t* lds = (lds_u8_t*)(smem);
  using L = Layout<kMode>;
  // Wave 0 builds them from the device offsets, clamped to [0, N_cap] (a
  // caller contract violation cannot push a row index outside the buffers):
  // lane l takes experts l * per .. l * per + per - 1 (per = ceil(E / 64) <= 16),
  // expert e gets ceil((max(hi, lo) - lo) / BM) row tiles, and a prefix of the
  // lane sums across the wave places them.
  if (threadIdx.x < kWave) {
    constexpr int kPer = kMaxExperts / kWave;
    const int ln = threadIdx.x;
    const int per = (E + kWave - 1) / kWave;
    const int e0 = std::min(E, ln * per);
    auto clamp_off = [&](int e) {
      return static_cast<int32_t>(std::min<int64_t>(std::max<int64_t>(offsets[e], 0), N_cap));
    };
    int32_t c[kPer + 1];
#pragma unroll
    for (int q = 0; q <= kPer; ++q) c[q] = (q <= per && e0 + q <= E) ? clamp_off(e0 + q) : 0;
    int32_t tiles[kPer];
    int32_t sum = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      int32_t t = 0;
      if (q < per && e0 + q < E) t = (std::max(c[q + 1], c[q]) - c[q] + BM - 1) / BM;
      tiles[q] = t;
      sum += t;
    }
    int32_t incl = sum;
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t v = __shfl_up(incl, o, kWave);
      if (ln >= o) incl += v;
    }
    int32_t run = incl - sum;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (q < per && e0 + q < E) {
        s_prefix[e0 + q] = run;
        s_offs[e0 + q] = c[q];
        run += tiles[q];
      }
    }
    if (ln == kWave - 1) s_prefix[E] = incl;
    if (ln == 0) s_offs[E] = std::max(clamp_off(E), clamp_off(E - 1));  // the last expert's end
  }
  __syncthreads();
  const int32_t* prefix = s_prefix;
  const int32_t* offs = s_offs;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave & 1;   // 64-row half of the tile
  const int wn = wave >> 1;  // B-column block

  using MD = Mode<kMode>;
  constexpr int kOutCols = MD::kPaired ? BN / 2 : BN;
  constexpr int kStoresPerTile = EpiloguePlan<kMode>::kStores;
  constexpr int kPreStores = EpiloguePlan<kMode>::kPreStores;
  static_assert(L::kLoadsPerStage + kStoresPerTile + kPreStores < 64, "vmcnt field is 6 bits");
  const bool keep_pre = kMode == 0 && preact != nullptr;
  const int col_tiles = (Ncols + kOutCols - 1) / kOutCols;
  const int row_tiles = prefix[E];
  const int total = row_tiles * col_tiles;  // < 2^31: at most (2^31 / 128 + 1024) * 32

  // XCD-aware split of the logical tile space: workgroup b runs on XCD b % 8.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = G / kXcds;
  const int t_lo = static_cast<int>(int64_t(total) * xcd / kXcds);
  const int t_hi = static_cast<int>(int64_t(total) * (xcd + 1) / kXcds);
  const int ksteps = Kdim / BK;

  // LDS byte offsets (within a stage) of this lane's B-operand transpose reads
  // for sub-step 0; sub-step kk adds 16 rows, which keeps k & 3 and the swizzle
  int b_off[L::kColFrags][2];  // [n-frag][half]
  const int g16 = lane / 16, i16 = lane % 16;
#pragma unroll
  for (int j = 0; j < L::kColFrags; ++j) {
    // gate/up: the first half of the blocks are gate columns, the second the
    // matching up columns
    constexpr int kHalf = L::kColFrags / 2;
    int ncol;
    if (MD::kPaired) ncol = (j < kHalf ? 0 : BN / 2) + wn * (BN / 2 / L::kWavesN) + (j % kHalf) * 32;
    else ncol = wn * (BN / L::kWavesN) + j * 32;
    const int n = ncol + 16 * (g16 % 2) + 4 * (i16 % 4);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = 8 * (g16 / 2) + i16 / 4 + 4 * half;  // + 16 * kk at use (k & 3 unchanged)
      b_off[j][half] = kChunksA * 16 + swz_b(k, n / 8) * 16 + (n % 8) * 2;
    }
  }

  // This workgroup's tiles: first, first + per_xcd, ... inside [t_lo, t_hi).
  // The k-steps of all of them form one sequence s = j * ksteps + ks, and the
  // loads run two steps ahead of the multiply across tile boundaries, so the
  // next tile's first stages are in flight during this tile's epilogue.
  const int first = t_lo + static_cast<int>(blockIdx.x) / kXcds;
  const int ntiles = uniform((first < t_hi) ? (t_hi - 1 - first) / per_xcd + 1 : 0);
  const int nsteps = ntiles * ksteps;

  struct TileInfo {
    int e, row0, row_end, n0;
  };
  auto tile_info = [&](int j) {
    const int tile = first + j * per_xcd;
    const int rt = tile / col_tiles;
    const int ct = tile - rt * col_tiles;
    // Expert owning row tile rt: the last e < E with prefix[e] <= rt (prefix
    // is non-decreasing and prefix[0] = 0, so the e that pass form a run from
    // 0). Two wave-wide probes instead of a binary search: lane l tests
    // e = 16 l (E <= 1024), then lanes 0..15 test the 16 e of the last block
    // that passed; the highest passing lane of each ballot gives the answer.
    const int e1 = 16 * lane;
    const uint64_t b1 = __builtin_amdgcn_ballot_w64(e1 < E && prefix[e1] <= rt);
    const int blk = 63 - __builtin_clzll(b1);
    const int e2 = 16 * blk + (lane & 15);
    const uint64_t b2 = __builtin_amdgcn_ballot_w64(lane < 16 && e2 < E && prefix[e2] <= rt);
    const int lo = uniform(16 * blk + 63 - __builtin_clzll(b2));
    TileInfo t;
    t.e = lo;
    t.row0 = offs[lo] + (rt - prefix[lo]) * BM;
    t.row_end = std::min(t.row0 + BM, offs[lo + 1]);
    t.n0 = ct * kOutCols;
    return t;
  };

  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  // Load cursor: tile index lj and k-step lk of the next stage to issue, with the
  // global sources of this thread's loads for tile lj precomputed (each k-step
  // only adds its k offset).
  int lj = 0;
  int lk = 0;
  int lbuf = 0;
  // A rows through a buffer resource that spans the tile's valid rows only: a
  // padding row (a tile past the end of its expert's rows) gets an offset past
  // the range, so its loads are issued and counted but move no data; what they
  // leave in LDS only reaches output rows that are never stored.
  uint32_t a_off[L::kLoadsA];
  i32x4_t a_rsrc;
  // B sources one k-step before the next load's (each load first advances
  // its pointer by one k-step of rows)
  const uint16_t* b_src[L::kLoadsB];
  const uint64_t b_adv = MD::kBkc ? uint64_t(BK) * 2 : uint64_t(BK) * Ncols * 2;
  auto load_tile_sources = [&](int j) {
    const TileInfo t = tile_info(j);
    const int rows = t.row_end - t.row0;
    a_rsrc = buffer_rsrc(A + int64_t(t.row0) * Kdim, static_cast<uint32_t>(rows * Kdim * 2));
#pragma unroll
    for (int i = 0; i < L::kLoadsA; ++i) {
      const int slot = i * L::kThreads + wave * kWave + lane;
      const int m = slot >> 3;
      const int kc = (slot & 7) ^ ((m >> 1) & 7);
      a_off[i] = m < rows ? static_cast<uint32_t>((m * Kdim + kc * 8) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < L::kLoadsB; ++i) {
      const int slot = i * L::kThreads + wave * kWave + lane;
      if (MD::kBkc) {
        // B_e rows n (k contiguous, ksplit per row in B0), stored like the A rows
        const int n = slot >> 3;
        const int kc = (slot & 7) ^ ((n >> 1) & 7);
        int ng = t.n0 + n;
        if (ng >= Ncols) ng = 0;  // rows past the matrix: any valid address, never stored
        b_src[i] = B0 + (int64_t(t.e) * Ncols + ng) * ksplit + kc * 8 - BK;
        continue;
      }
      const int k = slot >> 5;
      const int c = (slot & 31) ^ (4 * (k & 3));
      const uint16_t* base;
      int col;
      if (MD::kPaired) {
        base = (c < 16) ? B0 : B1;
        col = t.n0 + (c % 16) * 8;
      } else {
        base = B0;
        col = t.n0 + c * 8;
      }
      if (col >= Ncols) col = 0;  // columns past the matrix: any valid address, never stored
      b_src[i] = base + int64_t(t.e) * Kdim * Ncols + int64_t(k - BK) * Ncols + col;
    }
  };
  uint32_t l_st = 0;
  // kBkc: at the k-step where k reaches ksplit the B sources move from B0[e] to
  // the same rows of B1[e] (ksplit is a multiple of BK)
  const int lk_b1 = MD::kBkc ? ksplit / BK : -1;
  auto issue_begin = [&]() {
    if (lk == 0) {
      load_tile_sources(lj);
    } else if (MD::kBkc && lk == lk_b1) {
#pragma unroll
      for (int i = 0; i < L::kLoadsB; ++i) b_src[i] = B1 + ((b_src[i] - B0) - ksplit);
    }
    l_st = uniform(static_cast<int>(lds0 + lbuf * kStageBytes + wave * kWave * 16));
  };
  // load i (0 .. kLoadsPerStage - 1) of the stage being issued
  auto load1 = [&](int i) {
    if (i < L::kLoadsA)
      buffer_load_lds16_at(a_rsrc, a_off[i], uniform(lk * BK * 2), l_st, i * L::kThreads * 16);
    else
      global_load_lds16_step(b_src[i - L::kLoadsA], b_adv, l_st,
                             (kChunksA + (i - L::kLoadsA) * L::kThreads) * 16);
  };
  auto issue_end = [&]() {
    lbuf = (lbuf + 1 == kStages) ? 0 : lbuf + 1;
    if (++lk == ksteps) {
      lk = 0;
      ++lj;
    }
  };
  auto issue_next = [&]() {
    issue_begin();
#pragma unroll
    for (int i = 0; i < L::kLoadsPerStage; ++i) load1(i);
    issue_end();
  };

  // LDS read r (0 .. kReads - 1) of the fragments of sub-step kk: A row block
  // 0, the two halves of each B column block, A row block 1 (the order the
  // MFMAs use them)
  auto rd = [&](const lds_u8_t* st_, int kk_, int r, bf16x8_t* na, bf16x8_t* nb) {
    if (r == 0 || r == L::kReads - 1) {
      const int i = r == 0 ? 0 : 1;
      na[i] = lds_read_a(st_, swz(wm * 64 + i * 32 + lane % 32, kk_ * 2 + lane / 32));
    } else {
      const int jj = (r - 1) / 2, half = (r - 1) % 2;
      if (MD::kBkc) {
        // rows n of B_e, k-chunk kk * 2 + lane / 32: read like the A rows
        if (half == 0)
          nb[jj] = lds_read_a(st_ + kChunksA * 16,
                              swz(wn * (BN / L::kWavesN) + jj * 32 + lane % 32, kk_ * 2 + lane / 32));
      } else {
        const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(st_ + b_off[jj][half] + kk_ * 16 * (BN * 2)));
        __builtin_memcpy(reinterpret_cast<char*>(&nb[jj]) + 8 * half, &v, 8);
      }
    }
  };
  // Schedule of one k-step (one wave per SIMD, in-order issue: a wave issues
  // at most one instruction per issue turn, so non-MFMA instructions placed
  // between two MFMAs cost nothing while the matrix pipe is busy, and the same
  // instructions issued as a block leave it idle). Stage t's loads go out
  // during step t - 2 into the buffer that step t - 3 used (free since the
  // barrier that ended step t - 3's reads). In sub-steps 0..2 each MFMA is
  // followed by two of the ten LDS reads of the next sub-step's fragments (in
  // the order its MFMAs use them) or by this step's loads (sub-step 2 also
  // takes the last three). In sub-step 3 the wave runs two MFMAs, waits for
  // the next stage and passes the barrier, then follows each further MFMA with
  // two reads of the next stage's first fragments. sched_barrier pins this
  // order.
  int issued = 0;
  for (; issued < nsteps && issued < kStages - 1; ++issued) issue_next();
  bf16x8_t fa[2][2], fb[2][L::kColFrags];
  if (nsteps > 0) {
    if (issued > 1) wait_vmcnt<L::kLoadsPerStage>();
    else wait_vmcnt<0>();
    stage_barrier();
#pragma unroll
    for (int r = 0; r < L::kReads; ++r) rd(lds, 0, r, fa[0], fb[0]);
  }
  int s = 0;  // global k-step being multiplied
  int cbuf = 0;
  int epi_step = -8;  // k-step after which the last epilogue ran
  for (int j = 0; j < ntiles; ++j) {
    const TileInfo ci = tile_info(j);
    f32x16_t acc[2][L::kColFrags];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < L::kColFrags; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;
    auto mm = [&](int c, int i, int jj) {
      acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][jj], fa[c][i], acc[i][jj], 0, 0, 0);
    };

    // One k-step; kLoads (stage s + 2 goes out during this step) is a
    // template constant so the steady-state body carries no per-load branch.
    auto kstep_body = [&](auto loads_tag) {
      constexpr bool loads_now = decltype(loads_tag)::value;
      const lds_u8_t* st = lds + cbuf * kStageBytes;
      cbuf = (cbuf + 1 == kStages) ? 0 : cbuf + 1;
      const bool more = s + 1 < nsteps;
      if (loads_now) issue_begin();
      // One MFMA, then up to two LDS reads or one load: the non-MFMA
      // instructions of a sub-step issue in the shadows of its MFMAs.
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < BK / 16) {
          // reads of sub-step kk + 1 after MFMAs 0..4; this sub-step's loads
          // after MFMAs 5..7 (sub-step 2 also takes the last three)
#pragma unroll
          for (int m = 0; m < L::kMfmas; ++m) {
            mm(cur, m / L::kColFrags, m % L::kColFrags);
            __builtin_amdgcn_sched_barrier(0);
            if (m < L::kReads / 2) {
              rd(st, kk + 1, 2 * m, fa[cur ^ 1], fb[cur ^ 1]);
              rd(st, kk + 1, 2 * m + 1, fa[cur ^ 1], fb[cur ^ 1]);
            } else if (loads_now) {
              if (L::kWavesN == 2) {  // 12 loads: 3 in sub-steps 0 and 1, 6 in 2
                load1(3 * kk + (m - 5));
                if (kk == 2) load1(9 + (m - 5));
              } else {                // 6 loads: 2 per sub-step
                load1(2 * kk);
                load1(2 * kk + 1);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          // two MFMAs, then the stage hand-over, then the reads of the next
          // stage's first sub-step after MFMAs 2..6 (unconditional: after the
          // last step they read a stage nobody uses)
          mm(cur, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          mm(cur, 0, 1);
          __builtin_amdgcn_sched_barrier(0);
          wait_lds_reads();  // on every path: this wave is done reading stage s
          if (more) {
            // stage s + 2 is in flight: issued now, or earlier (never, once the
            // loads have run out)
            const bool next_loads = loads_now || issued > s + 2;
            if (epi_step != s - 1) {
              if (next_loads) wait_vmcnt<L::kLoadsPerStage>(); else wait_vmcnt<0>();
            } else if (keep_pre) {
              if (next_loads) wait_vmcnt<L::kLoadsPerStage + kStoresPerTile + kPreStores>();
              else wait_vmcnt<kStoresPerTile + kPreStores>();
            } else {
              if (next_loads) wait_vmcnt<L::kLoadsPerStage + kStoresPerTile>();
              else wait_vmcnt<kStoresPerTile>();
            }
            stage_barrier();  // everyone is done reading stage s; s + 1 is visible
          } else {
            // the workgroup's last k-step: the epilogue stages its output in
            // stage s, so every wave must be done reading it first
            stage_barrier();
          }
          __builtin_amdgcn_sched_barrier(0);
          const lds_u8_t* nst = lds + cbuf * kStageBytes;
          // reads per remaining MFMA: 2 (4 waves: 10 reads over 6 MFMAs) or
          // 3 (8 waves: 6 reads over 2 MFMAs)
          constexpr int kRpm = (L::kReads + L::kMfmas - 3) / (L::kMfmas - 2);
#pragma unroll
          for (int m = 2; m < L::kMfmas; ++m) {
            mm(cur, m / L::kColFrags, m % L::kColFrags);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = (m - 2) * kRpm; r < (m - 1) * kRpm && r < L::kReads; ++r)
              rd(nst, 0, r, fa[cur ^ 1], fb[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (loads_now) {
        issue_end();
        ++issued;
      }
    };
    // k-step s issues stage s + 2 while s + 2 < nsteps: in this tile the
    // first kload steps do, the rest (the workgroup's last two) do not
    const int kload = std::min(ksteps, std::max(0, nsteps - 2 - j * ksteps));
    int kstep = 0;
    for (; kstep < kload; ++kstep, ++s) kstep_body(std::true_type{});
    for (; kstep < ksteps; ++kstep, ++s) kstep_body(std::false_type{});

    epi_step = s - 1;
    {
      using EP = EpiloguePlan<kMode>;
      static_assert(L::kThreads / kWave * EP::kWaveStride <= kStageBytes,
                    "staging fits one ring stage");
      // Staging space: the ring stage of step s - 1, which every wave has
      // finished reading (the barrier of that step's last sub-step, taken on
      // the workgroup's last step too) and which is refilled only by stage
      // s + 2's loads, issued during step s after the barrier at the end of
      // this epilogue.
      lds_u8_t* stg = lds + ((cbuf + kStages - 1) % kStages) * kStageBytes + wave * EP::kWaveStride;
      constexpr int ldc = (kMode == 2 || kMode == 4) ? 2 : 1;  // C row stride in units of Ncols
      // Buffer stores: a store whose offset lies past the tile's last valid
      // row is dropped by the hardware, so padding rows need no branch and
      // every lane issues every store (the vmcnt waits count them).
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          C + int64_t(ci.row0) * Ncols * ldc, 0, (ci.row_end - ci.row0) * Ncols * ldc * 2,
          0x00020000);
      const int wcol0 = ci.n0 + (MD::kPaired ? wn * (BN / 2 / L::kWavesN) : wn * (BN / L::kWavesN));  // wave's first output column
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = lane % 32;  // this lane's row in the fragment
        const int row = ci.row0 + wm * 64 + i * 32 + r;
#pragma unroll
        for (int jj = 0; jj < EP::kOutFrags; ++jj) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wcol0 + jj * 32 + 8 * q + 4 * (lane / 32);
            float v[4], w[4];
            float d[4] = {0.f, 0.f, 0.f, 0.f};
            if (kMode == 2 && row < ci.row_end && col < Ncols) {
              const uint2 dh = *reinterpret_cast<const uint2*>(aux + int64_t(row) * Ncols + col);
              d[0] = bf16_lo(dh.x);
              d[1] = bf16_hi(dh.x);
              d[2] = bf16_lo(dh.y);
              d[3] = bf16_hi(dh.y);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if (kMode == 0) {
                const float g = acc[i][jj][4 * q + k];
                const float u = acc[i][jj + EP::kOutFrags][4 * q + k];
                v[k] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
              } else if (kMode == 2) {
                swiglu_grad(d[k], acc[i][jj][4 * q + k], acc[i][jj + EP::kOutFrags][4 * q + k],
                            &v[k], &w[k]);
              } else {
                v[k] = acc[i][jj][4 * q + k];
              }
            }
            // chunk of these four columns in the staged row, and which half of it
            const int chunk = 4 * jj + q;
            const u32x2_t pv = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                stg + r * EP::kRowBytes + stage_chunk<EP::kRowBytes>(r, chunk) * 16 +
                (lane / 32) * 8) = pv;
            if (kMode == 2) {  // du in the second half of the staged row
              const u32x2_t pw = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
              *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                  stg + r * EP::kRowBytes + stage_chunk<EP::kRowBytes>(r, EP::kChunks / 2 + chunk) * 16 +
                  (lane / 32) * 8) = pw;
            }
          }
        }
        // this wave's writes have landed before it reads them back (the
        // staging area is private to the wave)
        wait_lds_reads();
#pragma unroll
        for (int t = 0; t < EP::kStoresPerFrag; ++t) {
          const int rr = t * EP::kRowsPerStore + lane / EP::kChunks;
          const int c = lane % EP::kChunks;
          const u32x4_t val = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
              stg + rr * EP::kRowBytes + stage_chunk<EP::kRowBytes>(rr, c) * 16);
          const int lrow = wm * 64 + i * 32 + rr;  // row within the tile
          if (kMode == 4) {
            // eight bf16 dh values of one row: dg and du from the kept
            // pre-activations, each written as one 16-byte store
            const int col = wcol0 + c * 8;
            const bool ok = ci.row0 + lrow < ci.row_end && col < Ncols;
            u32x4_t dgv = {0u, 0u, 0u, 0u}, duv = {0u, 0u, 0u, 0u};
            if (ok) {
              const float* pg = preact + int64_t(ci.row0 + lrow) * (2 * Ncols) + col;
              const u32x4_t g0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg));
              const u32x4_t g1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + 4));
              const u32x4_t u0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + Ncols));
              const u32x4_t u1 =
                  __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + Ncols + 4));
              const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
              const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
              const uint32_t dw[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float dg0, du0, dg1, du1;
                swiglu_grad(bf16_lo(dw[q]), __uint_as_float(gw[2 * q]), __uint_as_float(uw[2 * q]),
                            &dg0, &du0);
                swiglu_grad(bf16_hi(dw[q]), __uint_as_float(gw[2 * q + 1]),
                            __uint_as_float(uw[2 * q + 1]), &dg1, &du1);
                dgv[q] = pack_bf16x2(dg0, dg1);
                duv[q] = pack_bf16x2(du0, du1);
              }
            }
            const int off = ok ? (lrow * 2 * Ncols + col) * 2 : 0x80000000;
            const int off2 = ok ? (lrow * 2 * Ncols + Ncols + col) * 2 : 0x80000000;
            __builtin_amdgcn_raw_buffer_store_b128(dgv, rsrc, off, 0, /*nt*/ 2);
            __builtin_amdgcn_raw_buffer_store_b128(duv, rsrc, off2, 0, /*nt*/ 2);
            continue;
          }
          int col, dst_col;
          if (kMode == 2) {
            col = wcol0 + (c % (EP::kChunks / 2)) * 8;
            dst_col = (c < EP::kChunks / 2) ? col : Ncols + col;
          } else {
            col = wcol0 + c * 8;
            dst_col = col;
          }
          const bool ok = ci.row0 + lrow < ci.row_end && col < Ncols;
          const int off = ok ? (lrow * Ncols * ldc + dst_col) * 2 : 0x80000000;
          // h and [dg | du] non-temporal (so they do not displace the operand
          // panels in L2); y plain, since the combine that follows reads it
          // back and finds it in the caches
          __builtin_amdgcn_raw_buffer_store_b128(val, rsrc, off, 0, kMode == 1 ? 0 : /*nt*/ 2);
        }
        if (kMode == 0 && keep_pre) {
          // g, then u, of this fragment (fp32, as the SwiGLU used them) through
          // the staging area as [32 rows][256 B], written back 4 rows x 256 B
          // per store into preact [N, 2 Ncols] (g at col, u at Ncols + col);
          // non-temporal, dropped past the tile's valid rows like the h stores
          const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
              preact + int64_t(ci.row0) * 2 * Ncols, 0, (ci.row_end - ci.row0) * 2 * Ncols * 4,
              0x00020000);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            // the staging area is free: this wave's reads of it have completed
            wait_lds_reads();
            const int r = lane % 32;
#pragma unroll
            for (int jj = 0; jj < EP::kOutFrags; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x16_t& a = acc[i][jj + half * EP::kOutFrags];
                const u32x4_t pv = {__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                                    __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
                const int chunk = 8 * jj + 2 * q + lane / 32;  // columns 4 chunk .. 4 chunk + 3
                *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(
                    stg + r * 256 + stage_chunk<256>(r, chunk) * 16) = pv;
              }
            wait_lds_reads();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int rr = 4 * t + lane / 16, c = lane % 16;
              const u32x4_t val = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                  stg + rr * 256 + stage_chunk<256>(rr, c) * 16);
              const int lrow = wm * 64 + i * 32 + rr;
              const int col = wcol0 + 4 * c;
              const bool ok = ci.row0 + lrow < ci.row_end && col < Ncols;
              const int off = ok ? (lrow * 2 * Ncols + half * Ncols + col) * 4 : 0x80000000;
              __builtin_amdgcn_raw_buffer_store_b128(val, prs, off, 0, /*nt*/ 2);
            }
          }
        }
      }
      // every wave has read its staged rows before stage s + 2's loads refill
      // this ring stage
      wait_lds_reads();
      stage_barrier();
    }
  }
}

}  // namespace

int persistent_grid() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return std::max(kXcds, (cus / kXcds) * kXcds);
}

// The forward builds its tile schedule in LDS and needs no workspace; the size
// (the 2 (E + 1) int32 that a separate schedule launch once wrote) is kept, so a
// workspace sized for it stays valid, and the backward's layout starts after it.
size_t gemm_workspace_bytes(int E, int64_t /*N_cap*/, int /*H*/, int /*I*/) {
  return ((static_cast<size_t>(2 * (E + 1)) * 4 + 255) / 256) * 256;
}

hipError_t launch_grouped_gemm_swiglu(const uint16_t* x, const int32_t* offsets, int E,
                                      int64_t N_cap, int H, int I, const uint16_t* wg,
                                      const uint16_t* wu, const uint16_t* wd, uint16_t* h,
                                      uint16_t* y, float* preact, void* /*ws*/, hipStream_t st) {
  if (N_cap == 0) return hipGetLastError();
  const int G = persistent_grid();
  hipLaunchKernelGGL(k_gemm<0>, dim3(G), dim3(Layout<0>::kThreads), 0, st, x, H, wg, wu, I,
                     offsets, E, N_cap, h, nullptr, preact, 0);
  hipLaunchKernelGGL(k_gemm<1>, dim3(G), dim3(Layout<1>::kThreads), 0, st, h, I, wd, nullptr, H,
                     offsets, E, N_cap, y, nullptr, nullptr, 0);
  return hipGetLastError();
}

// Backward: dh = dy Wd^T (row-grouped), [dg | du] from the recomputed gate/up
// tiles (mode 2), dx = [dg | du] [Wg ; Wu]^T (row-grouped), dWd = h^T dy and
// [dWg | dWu] = x^T [dg | du] (sums over each expert's rows). With the
// forward's fp32 pre-activations (preact) the gate/up GEMM is not run again:
// the dh GEMM's epilogue forms [dg | du] from them directly, with the same
// values and the same arithmetic as the recomputing path, so both paths give
// the same bits.
// ws layout: forward tables | backward tables | zeros[256 B]
//            | dh [N_cap, I] bf16 | dgu [N_cap, 2I] bf16
size_t gemm_grad_layout(int E, int64_t N_cap, int I, size_t* off_bt, size_t* off_zero,
                        size_t* off_dh, size_t* off_dgu) {
  const size_t fwd = ((gemm_workspace_bytes(E, N_cap, 0, 0) + 255) / 256) * 256;
  *off_bt = fwd;
  *off_zero = fwd + bgemm_sched_bytes(E);
  *off_dh = *off_zero + 256;
  *off_dgu = *off_dh + ((static_cast<size_t>(N_cap) * I * 2 + 255) / 256) * 256;
  return *off_dgu + static_cast<size_t>(N_cap) * 2 * I * 2;
}

size_t gemm_grad_workspace_bytes(int E, int64_t N_cap, int /*H*/, int I) {
  size_t a, b, c, d;
  return gemm_grad_layout(E, N_cap, I, &a, &b, &c, &d);
}

hipError_t launch_grouped_gemm_swiglu_grad(const uint16_t* x, const int32_t* offsets, int E,
                                           int64_t N_cap, int H, int I, const uint16_t* wg,
                                           const uint16_t* wu, const uint16_t* wd,
                                           const uint16_t* h, const uint16_t* dy, uint16_t* dx,
                                           uint16_t* dwg, uint16_t* dwu, uint16_t* dwd,
                                           const float* preact, void* ws, hipStream_t st) {
  size_t off_bt, off_zero, off_dh, off_dgu;
  gemm_grad_layout(E, N_cap, I, &off_bt, &off_zero, &off_dh, &off_dgu);
  char* base = static_cast<char*>(ws);
  int32_t* bt = reinterpret_cast<int32_t*>(base + off_bt);
  uint16_t* zeros = reinterpret_cast<uint16_t*>(base + off_zero);
  uint16_t* dh = reinterpret_cast<uint16_t*>(base + off_dh);
  uint16_t* dgu = reinterpret_cast<uint16_t*>(base + off_dgu);
  hipError_t err = launch_bgemm_sched(offsets, E, N_cap, bt, zeros, st);
  if (err != hipSuccess) return err;
  if (N_cap > 0) {
    const int G = persistent_grid();
    if (preact != nullptr) {
      // [dg | du] straight from the dh GEMM (dy Wd^T, B_e = Wd[e] stored [I][H])
      hipLaunchKernelGGL(k_gemm<4>, dim3(G), dim3(Layout<4>::kThreads), 0, st, dy, H, wd, wd, I,
                         offsets, E, N_cap, dgu, nullptr, const_cast<float*>(preact), H);
    } else {
      // dh = dy Wd^T (B_e = Wd[e] stored [I][H]), then [dg | du] from the
      // recomputed gate and up tiles
      hipLaunchKernelGGL(k_gemm<3>, dim3(G), dim3(Layout<3>::kThreads), 0, st, dy, H, wd, wd, I,
                         offsets, E, N_cap, dh, nullptr, nullptr, H);
      hipLaunchKernelGGL(k_gemm<2>, dim3(G), dim3(Layout<2>::kThreads), 0, st, x, H, wg, wu, I,
                         offsets, E, N_cap, dgu, dh, nullptr, 0);
    }
    // dx = [dg | du] [Wg ; Wu]^T: B_e = Wg[e], Wu[e] stored [H][I], side by side along k
    hipLaunchKernelGGL(k_gemm<3>, dim3(G), dim3(Layout<3>::kThreads), 0, st, dgu, 2 * I, wg, wu, H,
                       offsets, E, N_cap, dx, nullptr, nullptr, I);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // dWd = h^T dy  ([E, I, H]),  [dWg | dWu] = x^T [dg | du]  ([E, H, I] each)
  err = launch_bgemm_kgroup(h, I, I, dy, H, H, bt, E, zeros, dwd, dwd, H, H, st);
  if (err != hipSuccess) return err;
  return launch_bgemm_kgroup(x, H, H, dgu, 2 * I, 2 * I, bt, E, zeros, dwg, dwu, I, I, st);
}

}  // namespace moe
