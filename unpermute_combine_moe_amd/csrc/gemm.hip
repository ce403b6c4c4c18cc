// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Follows the twinkle grouped-matmul PR ("feat(moe): NPU平台 EP experts forward
// 计算改用 NPU grouped matmul"): every expert group of the expert-major buffer
// goes through one grouped matmul plus SwiGLU instead of a per-expert loop.
//   pass 1 (gate/up):  h = bf16( silu(x Wg[e]) * (x Wu[e]) )   fp32 accumulate
//   pass 2 (down):     y = bf16( h Wd[e] )                      fp32 accumulate
//
// Work decomposition. A small scheduling kernel turns the device-side expert
// offsets into a row-tile prefix (ceil(rows_e / BM) tiles per expert, 0 for an
// empty expert). Each GEMM pass is one persistent launch; a workgroup walks
// logical tiles (row tile, column tile) inside the range owned by its XCD, so
// the tiles that share an expert's weight panel and an A row-block run on the
// same XCD and reuse its L2.
//
// Tile: BM = 128 rows x 256 B-columns x BK = 64, 256 threads as 2 x 2 waves;
// each wave owns 64 rows x 128 B-columns = 2 x 4 MFMA 32x32 accumulators.
// Pass 1 packs 128 gate columns and the matching 128 up columns into the 256
// B-columns, so the SwiGLU epilogue finds g and u of an output element in the
// same lane and register. The weights are [K][N] (N contiguous); MFMA operands
// want 8 consecutive k per lane, so each thread loads an 8(k) x 8(n) block and
// transposes it in registers before writing it to LDS. LDS tiles are [row][k]
// in 16-byte chunks with the chunk index XOR-swizzled by (row & 7), which
// keeps both the transposed writes and the MFMA operand reads free of bank
// conflicts. Two LDS stages; the next k-step's global loads are in flight
// while the current one is multiplied.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 256;  // B-columns per tile
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kChunksA = BM * BK / 8;  // 16-byte chunks per stage
constexpr int kChunksB = BN * BK / 8;
constexpr int kSchedThreads = 1024;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int kc) { return row * (BK / 8) + (kc ^ (row & 7)); }

// ws layout (int32): tile_prefix[E+1] | offs[E+1]
__global__ void __launch_bounds__(kSchedThreads)
k_gemm_sched(const int32_t* __restrict__ offsets, int E, int64_t N_cap, int32_t* __restrict__ ws) {
  __shared__ int32_t part[kSchedThreads];
  int32_t* prefix = ws;
  int32_t* offs = ws + (E + 1);
  // clamped, non-decreasing offsets (a caller contract violation cannot push
  // a row index outside [0, N_cap])
  const int e = threadIdx.x;
  int32_t lo = 0, hi = 0;
  if (e < E) {
    lo = static_cast<int32_t>(std::min<int64_t>(std::max(offsets[e], 0), N_cap));
    hi = static_cast<int32_t>(std::min<int64_t>(std::max(offsets[e + 1], 0), N_cap));
    hi = std::max(hi, lo);
  }
  const int32_t tiles = (e < E) ? (hi - lo + BM - 1) / BM : 0;
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
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint4* base, int idx) {
  const uint4 v = base[idx];
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// kMode 0: gate/up + SwiGLU -> h.  kMode 1: down -> y.
template <int kMode>
__global__ void __launch_bounds__(kThreads, 1)
k_gemm(const uint16_t* __restrict__ A, int Kdim, const uint16_t* __restrict__ B0,
       const uint16_t* __restrict__ B1, int Ncols, const int32_t* __restrict__ ws, int E,
       uint16_t* __restrict__ C) {
  __shared__ uint4 sA[2][kChunksA];
  __shared__ uint4 sB[2][kChunksB];

  const int32_t* prefix = ws;
  const int32_t* offs = ws + (E + 1);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave & 1;   // 64-row half of the tile
  const int wn = wave >> 1;  // B-column half

  // columns of output produced per tile
  constexpr int kOutCols = (kMode == 0) ? BN / 2 : BN;
  const int col_tiles = (Ncols + kOutCols - 1) / kOutCols;
  const int row_tiles = prefix[E];
  const int64_t total = int64_t(row_tiles) * col_tiles;

  // XCD-aware split of the logical tile space: workgroup b runs on XCD b % 8.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = G / kXcds;
  const int64_t t_lo = total * xcd / kXcds;
  const int64_t t_hi = total * (xcd + 1) / kXcds;

  const int a_kc = tid % 8;        // A loader: chunk column and first row
  const int a_r0 = tid / 8;        // rows a_r0 + 32 i
  const int b_kg = tid % 8;        // B loader: 8-row k group
  const int b_ng = tid / 8;        // B loader: 8-column group 0..31
  const int ksteps = Kdim / BK;

  for (int64_t tile = t_lo + blockIdx.x / kXcds; tile < t_hi; tile += per_xcd) {
    const int rt = static_cast<int>(tile / col_tiles);
    const int ct = static_cast<int>(tile % col_tiles);
    // expert owning row tile rt: last e with prefix[e] <= rt
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (prefix[mid] <= rt) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = offs[e] + (rt - prefix[e]) * BM;
    const int row_end = std::min(row0 + BM, offs[e + 1]);
    const int n0 = ct * kOutCols;

    // A loader rows (clamped into the tile's valid rows; extra rows are never stored)
    const uint16_t* a_ptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = std::min(row0 + a_r0 + 32 * i, row_end - 1);
      a_ptr[i] = A + int64_t(r) * Kdim + a_kc * 8;
    }
    // B loader column base for this thread
    const uint16_t* b_ptr;
    bool b_valid;
    {
      int col;
      const uint16_t* base;
      if (kMode == 0) {
        base = (b_ng < 16) ? B0 : B1;
        col = n0 + (b_ng % 16) * 8;
      } else {
        base = B0;
        col = n0 + b_ng * 8;
      }
      b_valid = col < Ncols;
      b_ptr = base + int64_t(e) * Kdim * Ncols + int64_t(b_kg * 8) * Ncols + (b_valid ? col : 0);
    }

    Vec8 ra[4], rb[8];
    auto gload = [&](int ks) {
      const int64_t k0 = int64_t(ks) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = load16(a_ptr[i] + k0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b_valid) rb[j] = load16(b_ptr + (k0 + j) * Ncols);
        else rb[j] = Vec8{{0u, 0u, 0u, 0u}};
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = a_r0 + 32 * i;
        sA[buf][swz(r, a_kc)] = make_uint4(ra[i].w[0], ra[i].w[1], ra[i].w[2], ra[i].w[3]);
      }
      // 8x8 transpose: column c of the thread's block gets k = b_kg*8 .. +8
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int w = c >> 1;
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm(rb[1].w[w], rb[0].w[w], sel);
        o.y = __builtin_amdgcn_perm(rb[3].w[w], rb[2].w[w], sel);
        o.z = __builtin_amdgcn_perm(rb[5].w[w], rb[4].w[w], sel);
        o.w = __builtin_amdgcn_perm(rb[7].w[w], rb[6].w[w], sel);
        const int n = b_ng * 8 + c;
        sB[buf][swz(n, b_kg)] = o;
      }
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // B-column of each of the wave's four n-fragments
    int ncol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kMode == 0) ncol[j] = (j < 2 ? 0 : BN / 2) + wn * 64 + (j % 2) * 32 + lane % 32;
      else ncol[j] = wn * 128 + j * 32 + lane % 32;
    }
    int mrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) mrow[i] = wm * 64 + i * 32 + lane % 32;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < ksteps) gload(ks + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int kc = kk * 2 + lane / 32;
        bf16x8_t fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = lds_frag(sA[buf], swz(mrow[i], kc));
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = lds_frag(sB[buf], swz(ncol[j], kc));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (ks + 1 < ksteps) lstore(buf ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (row >= row_end) continue;
        if (kMode == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + lane % 32;
            if (col < Ncols) {
              const float g = acc[i][j][r];
              const float u = acc[i][j + 2][r];
              const float hv = g / (1.0f + __expf(-g)) * u;
              C[int64_t(row) * Ncols + col] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + j * 32 + lane % 32;
            if (col < Ncols)
              C[int64_t(row) * Ncols + col] = static_cast<uint16_t>(f32_to_bf16_rne(acc[i][j][r]));
          }
        }
      }
    }
  }
}

int persistent_grid() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return std::max(kXcds, (cus / kXcds) * kXcds);
}

}  // namespace

size_t gemm_workspace_bytes(int E, int64_t /*N_cap*/, int /*H*/, int /*I*/) {
  return static_cast<size_t>(2 * (E + 1)) * sizeof(int32_t);
}

hipError_t launch_grouped_gemm_swiglu(const uint16_t* x, const int32_t* offsets, int E,
                                      int64_t N_cap, int H, int I, const uint16_t* wg,
                                      const uint16_t* wu, const uint16_t* wd, uint16_t* h,
                                      uint16_t* y, void* ws, hipStream_t st) {
  int32_t* w = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_gemm_sched, dim3(1), dim3(kSchedThreads), 0, st, offsets, E, N_cap, w);
  if (N_cap == 0) return hipGetLastError();
  const int G = persistent_grid();
  hipLaunchKernelGGL(k_gemm<0>, dim3(G), dim3(kThreads), 0, st, x, H, wg, wu, I, w, E, h);
  hipLaunchKernelGGL(k_gemm<1>, dim3(G), dim3(kThreads), 0, st, h, I, wd, nullptr, H, w, E, y);
  return hipGetLastError();
}

}  // namespace moe
