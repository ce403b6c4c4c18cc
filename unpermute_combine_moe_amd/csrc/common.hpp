// Device helpers shared by the libmoeperm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kWave = 64;

// Below this many tokens the row kernels (permute rows, combine) give each
// token two waves, each taking every other 64-chunk row of the hidden dim: a
// wave per token would leave too few waves for several rounds on 1024 SIMDs.
constexpr int64_t kSplitBelowTokens = 16384;

// 16-byte vector of 8 bf16 values, moved as four dwords.
struct alignas(16) Vec8 {
  uint32_t w[4];
};

__device__ __forceinline__ Vec8 load16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return Vec8{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ void store16(void* p, const Vec8& v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}

// Non-temporal variants for streams that are written once and not re-read soon.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store16_nt(void* p, const Vec8& v) {
  u32x4_t u = {v.w[0], v.w[1], v.w[2], v.w[3]};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ Vec8 load16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return Vec8{{v.x, v.y, v.z, v.w}};
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const Vec8& v, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v.w[i]);
    f[2 * i + 1] = bf16_hi(v.w[i]);
  }
}

// fp32 -> bf16 bits, round to nearest, ties to even. NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even, by
// the gfx950 conversion instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t b = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

__device__ __forceinline__ Vec8 pack8(const float f[8]) {
  Vec8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// Correctly rounded bf16 of the exact product a*b where a is fp32 and b is a
// bf16 value (so the exact product has at most 32 significant bits). The
// fp32 product r is rounded once; its residual e = a*b - r is exact (fma).
// r can only sit on the wrong side of a bf16 rounding boundary when r lands
// exactly on a bf16 midpoint; the sign of e then decides the direction.
__device__ __forceinline__ uint32_t mul_to_bf16_exact(float a, float b) {
  const float r = a * b;
  const float e = __builtin_fmaf(a, b, -r);
  const uint32_t u = __float_as_uint(r);
  if ((u & 0xFFFFu) == 0x8000u && e != 0.0f && (u & 0x7F800000u) != 0x7F800000u) {
    // exact value is beyond the midpoint (away from zero) when e has r's sign
    const bool away = (e > 0.0f) == (r > 0.0f);
    return away ? ((u >> 16) + 1u) & 0xFFFFu : (u >> 16);
  }
  return f32_to_bf16_rne(r);
}

// Wave-uniform value (readfirstlane), for addresses the compiler should keep scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Wave-wide sum of a float (butterfly over all 64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// SwiGLU derivative for one element: with s = 1 / (1 + exp(-g)),
// dg = d u s (1 + g (1 - s)) and du = d g s. Every kernel that forms [dg | du]
// calls this one function, so the same g, u and d give the same bits.
__device__ __forceinline__ void swiglu_grad(float d, float g, float u, float* dg, float* du) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  *dg = d * u * s * (1.0f + g * (1.0f - s));
  *du = d * g * s;
}

// ---- staged-operand ring of the GEMM kernels

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16-byte direct global -> LDS load: this lane's 16 bytes land at LDS byte
// address lds_base + 16 * lane. Issued as inline asm so the compiler does not
// treat it as an LDS write it must wait for before every later LDS read; the
// kernel orders these loads itself with wait_vmcnt and stage_barrier.
__device__ __forceinline__ void load_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(gptr)
               : "memory", "m0");
}

// Raw buffer resource (gfx9 layout: base address, stride 0, num_records bytes,
// the same dword 3 the compiler's make_buffer_rsrc takes); every word made
// wave-uniform so the descriptor lives in SGPRs.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<uint32_t>(a)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(num_records));
  r.w = 0x00020000;
  return r;
}

// 16-byte direct buffer -> LDS load: this lane's 16 bytes (at byte voffset of
// the resource) land at LDS byte address lds_base + 16 * lane. An offset past
// the resource's num_records is out of range: the load moves no data but is
// issued and counted like any other, so the vmcnt bookkeeping is unchanged.
__device__ __forceinline__ void buffer_load_lds16(i32x4_t rsrc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence (a fence would also wait for the
// loads still in flight); the "memory" clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until this wave's own LDS accesses have completed.
__device__ __forceinline__ void wait_lds_reads() {
  // lgkmcnt(0); vmcnt (63) and expcnt (7) unconstrained
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Exclusive scan of in[0..L) into out[0..L) by one workgroup of kThreads
// threads (each a contiguous run, then a Hillis-Steele scan of the run sums in
// part[kThreads], shared); returns the total to every thread. in and out may
// alias. Every thread of the workgroup must call it.
template <int kThreads>
__device__ int32_t block_exclusive_scan(const int32_t* in, int32_t* out, int64_t L,
                                        int32_t* part) {
  const int64_t seg = ceil_div(L, kThreads);
  const int64_t lo = std::min<int64_t>(L, threadIdx.x * seg);
  const int64_t hi = std::min<int64_t>(L, lo + seg);
  int32_t sum = 0;
  for (int64_t i = lo; i < hi; ++i) sum += in[i];
  __syncthreads();
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int32_t v = static_cast<int>(threadIdx.x) >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - sum;
  const int32_t total = part[kThreads - 1];
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t c = in[i];
    out[i] = run;
    run += c;
  }
  __syncthreads();
  return total;
}

}  // namespace moe
