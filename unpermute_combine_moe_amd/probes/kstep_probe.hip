// Measurement aid (not part of the library): the forward grouped GEMM's
// k-step in isolation, on all 256 CUs, one workgroup of four waves per CU.
//
// The k-step is the gate/up pass's: a 128 x 256 tile, BK = 64, four waves of
// 64 x 128 (two A and four B fragments of v_mfma_f32_32x32x16_bf16 each), a
// three-stage ring of 48 KB in LDS with the same XOR swizzles, the B operand
// formed by ds_read_b64_tr_b16 transpose reads, the same MFMA order with the
// next sub-step's fragment reads after MFMAs 0..4 and the k-step's operand
// loads after MFMAs 5..7, one barrier per k-step. The ring holds random bf16
// values of magnitude 0.5..2 (so the MFMAs see operands like real data).
//
// Variants switch parts on or off (flags below). The operand loads, where on,
// read an L2-resident 48 KB buffer (every workgroup the same one), either
// straight into the ring stage being refilled (global_load_lds_dwordx4, as the
// GEMM does) or into registers that are written to that stage with
// ds_write_b128 at the end of the step. Each variant runs 4,096 k-steps twice;
// the line gives cycles per k-step (shader clock counter), the shader clock
// (cycles over the 100 MHz real-time counter) and ns per k-step.
//
// Build and run (from the repository root):
//   hipcc -std=c++17 -O3 --offload-arch=gfx950 -Xclang -target-feature \
//     -Xclang -packed-fp32-ops unpermute_combine_moe_amd/probes/kstep_probe.hip \
//     -o /tmp/kstep_probe && /tmp/kstep_probe
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kChunksA = BM * BK / 8, kChunksB = BN * BK / 8;
constexpr int kStageBytes = (kChunksA + kChunksB) * 16;
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kLoadsPerWave = 12;  // 48 KB per stage / (4 waves x 64 lanes x 16 B)
constexpr int kSrcElems = kStageBytes / 2;

// variant flags
constexpr int kMfma = 1;        // the MFMAs
constexpr int kReads = 2;       // the fragment reads
constexpr int kBarrier = 4;     // the per-k-step barrier
constexpr int kLdsLoads = 8;    // operand loads straight into LDS
constexpr int kRegLoads = 16;   // operand loads into registers, then ds_write_b128
constexpr int kBNMajor = 32;    // B stored n-major: one ds_read_b128 per B fragment
constexpr int kFull = kMfma | kReads | kBarrier;

__device__ __forceinline__ int swz(int row, int kc) { return row * (BK / 8) + (kc ^ ((row >> 1) & 7)); }
__device__ __forceinline__ int swz_b(int k, int c) { return k * (BN / 8) + (c ^ (4 * (k & 3))); }

__device__ __forceinline__ bf16x8_t read16(const lds_u8_t* base, int slot) {
  const u32x4_t v = *reinterpret_cast<const lds_u32x4_t*>(base + slot * 16);
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// lgkmcnt(0), other counters unconstrained (a form the compiler's own wait
// tracking understands)
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

__device__ __forceinline__ uint16_t random_bf16(uint32_t i) {
  uint32_t h = i * 2654435761u + 12345u;
  h ^= h >> 13;
  h *= 0x5bd1e995u;
  h ^= h >> 15;
  // sign, exponent 126..128 (magnitude 0.5 .. 2), random mantissa
  return static_cast<uint16_t>(((h & 1) << 15) | ((126 + (h >> 1) % 3) << 7) | ((h >> 3) & 127));
}

template <int kF>
__global__ void __launch_bounds__(kThreads, 1)
k_step(int nsteps, const uint16_t* __restrict__ src, float* __restrict__ out,
       unsigned long long* __restrict__ clk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_u8_t* lds = (lds_u8_t*)(smem);
  constexpr bool mfma = kF & kMfma, reads = kF & kReads, barrier = kF & kBarrier;
  constexpr bool lds_loads = kF & kLdsLoads, reg_loads = kF & kRegLoads, bn_major = kF & kBNMajor;
  for (int i = threadIdx.x; i < kStages * kStageBytes / 2; i += kThreads)
    reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(lds)[i] = random_bf16(i);
  __syncthreads();
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int kReadsPerSub = 10;  // 2 A fragments, 4 B fragments of two halves
  int b_off[4][2];
  {
    const int g16 = lane / 16, i16 = lane % 16;
    for (int j = 0; j < 4; ++j) {
      const int n = wn * 128 + j * 32 + 16 * (g16 % 2) + 4 * (i16 % 4);
      for (int half = 0; half < 2; ++half) {
        const int k = 8 * (g16 / 2) + i16 / 4 + 4 * half;
        b_off[j][half] = kChunksA * 16 + swz_b(k, n / 8) * 16 + (n % 8) * 2;
      }
    }
  }
  // read r of sub-step kk: A fragment 0, the halves of B fragments 0..3, A fragment 1
  auto rd = [&](const lds_u8_t* st, int kk, int r, bf16x8_t* na, bf16x8_t* nb) {
    if (r == 0 || r == kReadsPerSub - 1) {
      const int i = r == 0 ? 0 : 1;
      na[i] = read16(st, swz(wm * 64 + i * 32 + lane % 32, kk * 2 + lane / 32));
      return;
    }
    const int jj = (r - 1) / 2, half = (r - 1) % 2;
    if (bn_major) {
      if (half == 0)
        nb[jj] = read16(st + kChunksA * 16, swz(wn * 128 + jj * 32 + lane % 32, kk * 2 + lane / 32));
      return;
    }
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(st + b_off[jj][half] + kk * 16 * (BN * 2)));
    __builtin_memcpy(reinterpret_cast<char*>(&nb[jj]) + 8 * half, &v, 8);
  };
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  // load i of this wave into ring stage `stage` (straight to LDS); the source
  // alternates between two copies of the 48 KB buffer so no load is loop-invariant
  auto load_lds = [&](int stage, int i, int s) {
    const uint16_t* g = src + (s & 1) * kSrcElems + (i * kThreads + wave * 64 + lane) * 8;
    const uint32_t m = lds0 + stage * kStageBytes + (i * kThreads + wave * 64) * 16;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(m))
                 : "memory", "m0");
  };
  u32x4_t staged[kLoadsPerWave];
  auto load_reg = [&](int i, int s) {
    staged[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
        src + (s & 1) * kSrcElems + (i * kThreads + wave * 64 + lane) * 8));
  };
  if (lds_loads) {
    for (int i = 0; i < kLoadsPerWave; ++i) load_lds(0, i, 0);
    for (int i = 0; i < kLoadsPerWave; ++i) load_lds(1, i, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  f32x16_t acc[2][4];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8_t fa[2][2], fb[2][4];
  for (int r = 0; r < kReadsPerSub; ++r) {
    rd(lds, 0, r, fa[0], fb[0]);
    rd(lds, 1, r, fa[1], fb[1]);
  }
  uint32_t xsum = 0;
  auto mm = [&](int c, int i, int jj) {
    if (mfma) {
      acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][jj], fa[c][i], acc[i][jj], 0, 0, 0);
    } else {
      // keep the fragments live without the matrix pipe
      u32x4_t a, b;
      __builtin_memcpy(&a, &fa[c][i], 16);
      __builtin_memcpy(&b, &fb[c][jj], 16);
      xsum += a.x + a.y + a.z + a.w + b.x + b.y + b.z + b.w;
    }
  };
  wait_lds();
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  asm volatile("" ::"s"(t0), "s"(r0));  // both counters read before the loop
  int cbuf = 0;
  for (int s = 0; s < nsteps; ++s) {
    const lds_u8_t* st = lds + cbuf * kStageBytes;
    cbuf = cbuf + 1 == kStages ? 0 : cbuf + 1;
    const int refill = cbuf + 1 == kStages ? 0 : cbuf + 1;  // stage s + 2's buffer
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          mm(cur, m / 4, m % 4);
          __builtin_amdgcn_sched_barrier(0);
          if (reads && m < kReadsPerSub / 2) {
            rd(st, kk + 1, 2 * m, fa[cur ^ 1], fb[cur ^ 1]);
            rd(st, kk + 1, 2 * m + 1, fa[cur ^ 1], fb[cur ^ 1]);
          } else if (m >= 5 && (lds_loads || reg_loads)) {
            // 12 loads: 3 in sub-steps 0 and 1, 6 in sub-step 2
            const int i = 3 * kk + (m - 5);
            if (lds_loads) load_lds(refill, i, s); else load_reg(i, s);
            if (kk == 2) {
              if (lds_loads) load_lds(refill, 9 + (m - 5), s); else load_reg(9 + (m - 5), s);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        mm(cur, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mm(cur, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (lds_loads) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        if (reg_loads) {
#pragma unroll
          for (int i = 0; i < kLoadsPerWave; ++i)
            *reinterpret_cast<lds_u32x4_t*>(lds + refill * kStageBytes +
                                            (i * kThreads + wave * 64 + lane) * 16) = staged[i];
        }
        wait_lds();
        if (barrier) asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const lds_u8_t* nst = lds + cbuf * kStageBytes;
#pragma unroll
        for (int m = 2; m < 8; ++m) {
          mm(cur, m / 4, m % 4);
          __builtin_amdgcn_sched_barrier(0);
          if (reads) {
#pragma unroll
            for (int r = (m - 2) * 2; r < (m - 1) * 2 && r < kReadsPerSub; ++r)
              rd(nst, 0, r, fa[cur ^ 1], fb[cur ^ 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = static_cast<float>(xsum);
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[blockIdx.x * kThreads + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// The same work per k-step (4.19 MFLOP per workgroup) as a 256 x 256 tile
// with BK = 32: four waves of 128 x 128 (four A and four B fragments each,
// 256 accumulator registers), a four-stage ring of 32 KB (A rows of 64 bytes,
// B rows of 512 bytes), the loads of stage s + 3 issued during step s. Per
// k-step LDS carries 32 KB of loads and 64 KB of fragment reads instead of 48
// and 96.
constexpr int kStage2 = 32 * 1024;
constexpr int kStages2 = 4;
__device__ __forceinline__ int swz2(int row, int kc) { return row * 4 + (kc ^ ((row >> 1) & 3)); }

template <int kF>
__global__ void __launch_bounds__(kThreads, 1)
k_step_256(int nsteps, const uint16_t* __restrict__ src, float* __restrict__ out,
           unsigned long long* __restrict__ clk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_u8_t* lds = (lds_u8_t*)(smem);
  constexpr bool mfma = kF & kMfma, reads = kF & kReads, loads = kF & kLdsLoads;
  for (int i = threadIdx.x; i < kStages2 * kStage2 / 2; i += kThreads)
    reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(lds)[i] = random_bf16(i);
  __syncthreads();
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int kAOff = 0, kBOff = 16 * 1024;
  int b_off[4][2];
  {
    const int g16 = lane / 16, i16 = lane % 16;
    for (int j = 0; j < 4; ++j) {
      const int n = wn * 128 + j * 32 + 16 * (g16 % 2) + 4 * (i16 % 4);
      for (int half = 0; half < 2; ++half) {
        const int k = 8 * (g16 / 2) + i16 / 4 + 4 * half;
        b_off[j][half] = kBOff + swz_b(k, n / 8) * 16 + (n % 8) * 2;
      }
    }
  }
  // read r (0..11) of sub-step kk: A fragments 0..3, then the halves of B fragments 0..3
  auto rd = [&](const lds_u8_t* st, int kk, int r, bf16x8_t* na, bf16x8_t* nb) {
    if (r < 4) {
      na[r] = read16(st + kAOff, swz2(wm * 128 + r * 32 + lane % 32, kk * 2 + lane / 32));
      return;
    }
    const int jj = (r - 4) / 2, half = (r - 4) % 2;
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(st + b_off[jj][half] + kk * 16 * (BN * 2)));
    __builtin_memcpy(reinterpret_cast<char*>(&nb[jj]) + 8 * half, &v, 8);
  };
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  auto load_lds = [&](int stage, int i, int s) {  // i = 0..7
    const uint16_t* g = src + (s & 1) * kSrcElems + (i * kThreads + wave * 64 + lane) * 8;
    const uint32_t m = lds0 + stage * kStage2 + (i * kThreads + wave * 64) * 16;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(m))
                 : "memory", "m0");
  };
  if (loads) {
    for (int st = 0; st < 3; ++st)
      for (int i = 0; i < 8; ++i) load_lds(st, i, st);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  f32x16_t acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8_t fa[2][4], fb[2][4];
  for (int r = 0; r < 12; ++r) {
    rd(lds, 0, r, fa[0], fb[0]);
    rd(lds, 1, r, fa[1], fb[1]);
  }
  uint32_t xsum = 0;
  auto mm = [&](int c, int i, int jj) {
    if (mfma) {
      acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][jj], fa[c][i], acc[i][jj], 0, 0, 0);
    } else {
      u32x4_t a, b;
      __builtin_memcpy(&a, &fa[c][i], 16);
      __builtin_memcpy(&b, &fb[c][jj], 16);
      xsum += a.x + a.y + a.z + a.w + b.x + b.y + b.z + b.w;
    }
  };
  wait_lds();
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  asm volatile("" ::"s"(t0), "s"(r0));
  int cbuf = 0;
  for (int s = 0; s < nsteps; ++s) {
    const lds_u8_t* st = lds + cbuf * kStage2;
    const int refill = cbuf == 0 ? kStages2 - 1 : cbuf - 1;  // stage s + 3 = stage s - 1's buffer
    cbuf = cbuf + 1 == kStages2 ? 0 : cbuf + 1;
    // sub-step 0: the reads of sub-step 1 after MFMAs 0..5, the loads after MFMAs 6..13
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      mm(0, m / 4, m % 4);
      __builtin_amdgcn_sched_barrier(0);
      if (reads && m < 6) {
        rd(st, 1, 2 * m, fa[1], fb[1]);
        rd(st, 1, 2 * m + 1, fa[1], fb[1]);
      } else if (loads && m >= 6 && m < 14) {
        load_lds(refill, m - 6, s);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 1: two MFMAs, the hand-over, then the next stage's first reads
    mm(1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mm(1, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (loads) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    wait_lds();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const lds_u8_t* nst = lds + cbuf * kStage2;
#pragma unroll
    for (int m = 2; m < 16; ++m) {
      mm(1, m / 4, m % 4);
      __builtin_amdgcn_sched_barrier(0);
      if (reads && m < 8) {
        rd(nst, 0, 2 * (m - 2), fa[0], fb[0]);
        rd(nst, 0, 2 * (m - 2) + 1, fa[0], fb[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = static_cast<float>(xsum);
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[blockIdx.x * kThreads + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

template <int kF>
void run(const char* name, int grid, int nsteps, const uint16_t* src, float* out,
         unsigned long long* clk) {
  check(hipFuncSetAttribute(reinterpret_cast<const void*>(k_step<kF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kStages * kStageBytes),
        "hipFuncSetAttribute");
  for (int rep = 0; rep < 2; ++rep) {
    hipEvent_t a, b;
    check(hipEventCreate(&a), "hipEventCreate");
    check(hipEventCreate(&b), "hipEventCreate");
    check(hipEventRecord(a), "hipEventRecord");
    hipLaunchKernelGGL(k_step<kF>, dim3(grid), dim3(kThreads), kStages * kStageBytes, 0, nsteps,
                       src, out, clk);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(b), "hipEventRecord");
    check(hipEventSynchronize(b), "hipEventSynchronize");
    float ms = 0.f;
    check(hipEventElapsedTime(&ms, a, b), "hipEventElapsedTime");
    std::vector<unsigned long long> c(2 * grid);
    check(hipMemcpy(c.data(), clk, c.size() * sizeof(c[0]), hipMemcpyDeviceToHost), "hipMemcpy");
    double cy = 0, rt = 0;
    for (int i = 0; i < grid; ++i) {
      cy += c[2 * i];
      rt += c[2 * i + 1];
    }
    cy /= grid;
    rt /= grid;
    std::printf("%-58s %6.3f ms  %7.1f cycles/k-step  %.2f GHz  %5.0f ns/k-step\n", name, ms,
                cy / nsteps, cy / rt * 0.1, rt * 10.0 / nsteps);
    std::fflush(stdout);
    check(hipEventDestroy(a), "hipEventDestroy");
    check(hipEventDestroy(b), "hipEventDestroy");
  }
}


template <int kF>
void run256(const char* name, int grid, int nsteps, const uint16_t* src, float* out,
            unsigned long long* clk) {
  check(hipFuncSetAttribute(reinterpret_cast<const void*>(k_step_256<kF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kStages2 * kStage2),
        "hipFuncSetAttribute");
  for (int rep = 0; rep < 2; ++rep) {
    hipEvent_t a, b;
    check(hipEventCreate(&a), "hipEventCreate");
    check(hipEventCreate(&b), "hipEventCreate");
    check(hipEventRecord(a), "hipEventRecord");
    hipLaunchKernelGGL(k_step_256<kF>, dim3(grid), dim3(kThreads), kStages2 * kStage2, 0, nsteps,
                       src, out, clk);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(b), "hipEventRecord");
    check(hipEventSynchronize(b), "hipEventSynchronize");
    float ms = 0.f;
    check(hipEventElapsedTime(&ms, a, b), "hipEventElapsedTime");
    std::vector<unsigned long long> c(2 * grid);
    check(hipMemcpy(c.data(), clk, c.size() * sizeof(c[0]), hipMemcpyDeviceToHost), "hipMemcpy");
    double cy = 0, rt = 0;
    for (int i = 0; i < grid; ++i) {
      cy += c[2 * i];
      rt += c[2 * i + 1];
    }
    cy /= grid;
    rt /= grid;
    std::printf("%-58s %6.3f ms  %7.1f cycles/k-step  %.2f GHz  %5.0f ns/k-step\n", name, ms,
                cy / nsteps, cy / rt * 0.1, rt * 10.0 / nsteps);
    std::fflush(stdout);
    check(hipEventDestroy(a), "hipEventDestroy");
    check(hipEventDestroy(b), "hipEventDestroy");
  }
}

}  // namespace

int main() {
  const int grid = 256, nsteps = 4096;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  uint16_t* src = nullptr;
  check(hipMalloc(&out, grid * kThreads * sizeof(float)), "hipMalloc");
  check(hipMalloc(&clk, 2 * grid * sizeof(unsigned long long)), "hipMalloc");
  check(hipMalloc(&src, 2 * kSrcElems * sizeof(uint16_t)), "hipMalloc");
  {
    std::vector<uint16_t> h(2 * kSrcElems);
    for (int i = 0; i < 2 * kSrcElems; ++i) {
      uint32_t x = static_cast<uint32_t>(i % kSrcElems) * 2654435761u;
      x ^= x >> 15;
      h[i] = static_cast<uint16_t>(((x & 1) << 15) | ((126 + (x >> 1) % 3) << 7) | ((x >> 3) & 127));
    }
    check(hipMemcpy(src, h.data(), h.size() * sizeof(uint16_t), hipMemcpyHostToDevice), "hipMemcpy");
  }
  run<kMfma>("MFMAs only (operands in registers)", grid, nsteps, src, out, clk);
  run<kReads | kBarrier>("fragment reads only", grid, nsteps, src, out, clk);
  run<kFull>("MFMAs + fragment reads + barrier", grid, nsteps, src, out, clk);
  run<kMfma | kReads>("MFMAs + fragment reads, no barrier", grid, nsteps, src, out, clk);
  run<kBarrier | kLdsLoads>("direct-to-LDS loads only (+ waits, barrier)", grid, nsteps, src, out, clk);
  run<kReads | kBarrier | kLdsLoads>("fragment reads + direct-to-LDS loads", grid, nsteps, src, out, clk);
  run<kFull | kLdsLoads>("whole k-step, direct-to-LDS loads", grid, nsteps, src, out, clk);
  run<kFull | kBNMajor>("MFMAs + reads + barrier, B n-major (b128 reads)", grid, nsteps, src, out, clk);
  run<kFull | kLdsLoads | kBNMajor>("whole k-step, direct-to-LDS loads, B n-major", grid, nsteps, src, out, clk);
  run<kFull | kRegLoads>("whole k-step, loads into registers + ds_write_b128", grid, nsteps, src, out, clk);
  run256<kMfma | kReads>("256 x 256 tile, BK 32: MFMAs + fragment reads + barrier", grid, nsteps, src, out, clk);
  run256<kReads | kLdsLoads>("256 x 256 tile, BK 32: fragment reads + direct-to-LDS loads", grid, nsteps, src, out, clk);
  run256<kMfma | kReads | kLdsLoads>("256 x 256 tile, BK 32: whole k-step", grid, nsteps, src, out, clk);
  return 0;
}
