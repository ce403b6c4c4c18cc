// Backward of the weighted top-K combine with zero / copy / constant experts
// and the shared term: the adjoint of out[t] = sum_k p[t,k] v_k(t) + shared[t]
// for a given g = d out.
//
// Follows the torch_npu.npu_moe_distribute_combine_v2 page, 计算公式 (the
// combine sum; Moe(ori_x) = 0, ori_x and alpha_1*ori_x + alpha_2*v for the
// zero, copy and constant experts) and 参数说明 (the shared expert carries no
// weight, so its gradient is g itself and needs no kernel).
//
// Three kernels:
//  - k_combine_grad: one wave per token, everything that belongs to one token:
//    the expert-row gradients p*g (correctly rounded bf16), the per-slot
//    d_probs dot products, d_ori_x (copy and const slots), and d_alpha when
//    every token owns its own alpha elements (per-token layouts).
//  - k_const_grad_partial: the sums over tokens -- d_const_v[c,h] and d_alpha
//    for layouts shared by all tokens -- as fp32 partials of token segments,
//    one wave per (segment, 512-wide hidden tile, group of 4 const experts).
//  - k_const_grad_reduce / k_alpha_grad_reduce: add the segment partials in a
//    fixed order. No atomics: the result does not depend on scheduling.
// For per-token alpha and K <= 8 the first two run as one launch
// (k_combine_grad_with_partials), the partial sums beside the per-token work.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kConstGroup = 4;     // const experts per partial-sum wave
constexpr int kTileH = 8 * kWave;  // hidden elements per partial-sum wave
constexpr int kMaxSegments = 128;

enum SlotKind : int { kDrop = 0, kRow = 1, kCopy = 2, kConst = 3 };

// kAlphaPerH: the const-expert coefficients vary along h (stride_h != 0).
// kMaxK: the slot arrays are sized for K <= kMaxK (8 or 16), so that the
// common K <= 8 keeps half the registers; there the kernel is held to four
// waves per SIMD (at most 128 VGPRs, which it fits without spilling).
// The per-token body, for workgroup `block` of the per-token grid.
template <bool kHasRowMap, bool kAlphaPerH, int kMaxK>
__device__ __forceinline__ void combine_grad_tokens(
    int block, const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ expert_out,
    int64_t N, const int32_t* __restrict__ row_of_slot, const int32_t* __restrict__ row_map,
    const int32_t* __restrict__ ids, const float* __restrict__ probs, SlotMask mk, int64_t T,
    int K, int H, int E, SpecialArgs sp, CombineGradArgs o, int alpha_token, int nsplit) {
  // nsplit waves (1, 2 or 4) share a token, each taking every nsplit-th
  // 64-chunk row of the hidden dim; their per-slot sums meet in LDS
  __shared__ float xch[kWaves][2][kMaxK];
  const int w = threadIdx.x / kWave;
  const int part = w % nsplit;
  const int64_t t = uniform(static_cast<int>(block * (kWaves / nsplit) + w / nsplit));
  const bool live = t < T;
  if (nsplit == 1 && !live) return;
  const int lane = threadIdx.x % kWave;
  const int64_t copy_lo = int64_t(E) + sp.num_zero;
  const int64_t const_lo = copy_lo + sp.num_copy;
  const int64_t id_hi = const_lo + sp.num_const;

  // slot metadata, lane k for slot k (zero experts and dropped slots: kDrop)
  int m_kind = kDrop, m_src = 0;
  float m_p = 0.f, m_a1 = 0.f, m_a2 = 0.f;
  if (live && lane < K) {
    const int64_t s = t * K + lane;
    const int id_in = ids[s];
    const int id = mk.active(s) ? id_in : -1;  // a slot outside the mask is dropped
    m_p = probs[s];
    if (id >= 0 && id < E) {
      int64_t row = row_of_slot[s];
      if (kHasRowMap && row >= 0 && row < N) row = row_map[row];
      if (row >= 0 && row < N) {
        m_kind = kRow;
        m_src = static_cast<int>(row);
      }
    } else if (id >= copy_lo && id < const_lo) {
      m_kind = kCopy;
    } else if (id >= const_lo && id < id_hi) {
      m_kind = kConst;
      m_src = static_cast<int>(id - const_lo);
      if (!kAlphaPerH) {
        const int64_t ai = t * sp.a_st + int64_t(m_src) * sp.a_sc;
        m_a1 = sp.alpha1[ai];
        m_a2 = sp.alpha2[ai];
      }
    }
  }
  int kind[kMaxK], src[kMaxK];
  float p[kMaxK], a1[kMaxK], a2[kMaxK];
  bool need_ori = false;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    kind[k] = k < K ? __builtin_amdgcn_readlane(m_kind, k) : kDrop;
    src[k] = __builtin_amdgcn_readlane(m_src, k);
    p[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_p), k));
    a1[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_a1), k));
    a2[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_a2), k));
    need_ori |= kind[k] == kCopy || kind[k] == kConst;
  }

  // s1[k]: <g, row> for routed slots, <g, ori_x> for copy / const slots (the
  // whole <g, a1*ori_x + a2*v> when alpha varies along h); s2[k]: <g, v>.
  float s1[kMaxK], s2[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) s1[k] = s2[k] = 0.f;
  const int chunks = live ? H / 8 : 0;
  const uint16_t* grow = grad_out + t * H;
  const uint16_t* orow = need_ori ? sp.ori_x + t * H : nullptr;
  for (int c = lane + part * kWave; c < chunks; c += kWave * nsplit) {
    const int h0 = c * 8;
    Vec8 v[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (kind[k] == kRow) v[k] = load16_nt(expert_out + int64_t(src[k]) * H + h0);
    float g[8], x[8], dori[8];
    unpack8(load16_nt(grow + h0), g);
    if (need_ori) unpack8(load16(orow + h0), x);
#pragma unroll
    for (int i = 0; i < 8; ++i) dori[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (kind[k] == kRow) {
        float f[8];
        unpack8(v[k], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) s1[k] = __builtin_fmaf(g[i], f[i], s1[k]);
        if (o.d_expert_out != nullptr) {
          Vec8 d;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            d.w[i] = mul_to_bf16_exact(p[k], g[2 * i]) |
                     (mul_to_bf16_exact(p[k], g[2 * i + 1]) << 16);
          store16(o.d_expert_out + int64_t(src[k]) * H + h0, d);
        }
      } else if (kind[k] == kCopy) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s1[k] = __builtin_fmaf(g[i], x[i], s1[k]);
          dori[i] = __builtin_fmaf(p[k], g[i], dori[i]);
        }
      } else if (kind[k] == kConst) {
        float cv[8];
        unpack8(load16(sp.const_v + int64_t(src[k]) * H + h0), cv);
        if (kAlphaPerH) {
          const int64_t abase = t * sp.a_st + int64_t(src[k]) * sp.a_sc;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int64_t ai = abase + int64_t(h0 + i) * sp.a_sh;
            const float A1 = sp.alpha1[ai], A2 = sp.alpha2[ai];
            s1[k] = __builtin_fmaf(g[i], A1 * x[i] + A2 * cv[i], s1[k]);
            dori[i] = __builtin_fmaf(p[k] * A1, g[i], dori[i]);
          }
        } else {
          const float pa1 = p[k] * a1[k];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            s1[k] = __builtin_fmaf(g[i], x[i], s1[k]);
            s2[k] = __builtin_fmaf(g[i], cv[i], s2[k]);
            dori[i] = __builtin_fmaf(pa1, g[i], dori[i]);
          }
        }
      }
    }
    if (o.d_ori_x != nullptr) store16(o.d_ori_x + t * H + h0, pack8(dori));
  }

  // per-slot sums across the wave, then across the token's waves (the
  // partner's sums are added in part order); lane k keeps slot k's d_probs
  float r1[kMaxK], r2[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    r1[k] = r2[k] = 0.f;
    if (kind[k] == kDrop) continue;
    r1[k] = wave_sum(s1[k]);
    if (!kAlphaPerH && kind[k] == kConst) r2[k] = wave_sum(s2[k]);
  }
  if (nsplit > 1) {
    if (part != 0 && lane == 0) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        xch[w][0][k] = r1[k];
        xch[w][1][k] = r2[k];
      }
    }
    __syncthreads();
    if (part != 0 || !live) return;
    for (int q = 1; q < nsplit; ++q)  // partners in part order
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        r1[k] += xch[w + q][0][k];
        r2[k] += xch[w + q][1][k];
      }
  }
  float mine = 0.f;
  float pr1[kMaxK], pr2[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    pr1[k] = pr2[k] = 0.f;
    float val = r1[k];
    if (!kAlphaPerH && kind[k] == kConst) {
      val = a1[k] * r1[k] + a2[k] * r2[k];
      pr1[k] = p[k] * r1[k];
      pr2[k] = p[k] * r2[k];
    }
    if (lane == k) mine = kind[k] == kDrop ? 0.f : val;
  }
  if (lane < K) o.d_probs[t * K + lane] = mine;

  // alpha owned by this token: element (t, c) for every const expert c (one
  // element when the layout does not separate c); absent experts get 0
  if (!kAlphaPerH && alpha_token) {
    const int n_el = sp.a_sc == 0 ? 1 : sp.num_const;
    for (int c = lane; c < n_el; c += kWave) {
      float v1 = 0.f, v2 = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (kind[k] == kConst && (sp.a_sc == 0 || src[k] == c)) {
          v1 += pr1[k];
          v2 += pr2[k];
        }
      const int64_t ai = t * sp.a_st + int64_t(c) * sp.a_sc;
      if (o.d_alpha1 != nullptr) o.d_alpha1[ai] = v1;
      if (o.d_alpha2 != nullptr) o.d_alpha2[ai] = v2;
    }
  }
}

template <bool kHasRowMap, bool kAlphaPerH, int kMaxK>
__global__ void __launch_bounds__(kWaves * kWave)
__attribute__((amdgpu_waves_per_eu(kMaxK <= 8 ? 4 : 1)))
k_combine_grad(const uint16_t* __restrict__ grad_out, const uint16_t* __restrict__ expert_out,
               int64_t N, const int32_t* __restrict__ row_of_slot,
               const int32_t* __restrict__ row_map, const int32_t* __restrict__ ids,
               const float* __restrict__ probs, SlotMask mk, int64_t T, int K, int H, int E,
               SpecialArgs sp, CombineGradArgs o, int alpha_token, int nsplit) {
  combine_grad_tokens<kHasRowMap, kAlphaPerH, kMaxK>(
      static_cast<int>(blockIdx.x), grad_out, expert_out, N, row_of_slot, row_map, ids, probs, mk,
      T, K, H, E, sp, o, alpha_token, nsplit);
}

struct Partials {
  float* cv;  // [nseg][num_const][H]: sum of p * alpha2 * g
  float* a1;  // [nseg][num_const][H]: sum of p * g * ori_x   (kSharedAlpha only)
  float* a2;  // [nseg][num_const][H]: sum of p * g * const_v (kSharedAlpha only)
  int nseg;
  int64_t seg_len;
};

// Slots scanned per round of the partial-sum kernel (8 per lane, loaded
// together), and const slots whose row loads are issued together.
constexpr int kRoundSlots = 8 * kWave;
template <bool kSharedAlpha>
constexpr int batch_slots() { return kSharedAlpha ? 4 : 8; }

// One wave per (token segment, hidden tile, const group). Each round loads
// the ids / probs of up to 512 slots at once, compacts the slots of this
// const group into an LDS list (wave-private), then walks the list in
// batches whose grad_out (and ori_x, const_v, alpha) loads are all in flight
// together.
// The partial-sum body, for workgroup (bx, by, bz) of the partial-sum grid.
template <bool kAlphaPerH, bool kSharedAlpha>
__device__ __forceinline__ void const_grad_partial_block(
    int bx, int by, int bz, const uint16_t* __restrict__ grad_out,
    const int32_t* __restrict__ ids, const float* __restrict__ probs, SlotMask mk, int64_t T,
    int K, int H, int E, SpecialArgs sp, Partials part) {
  constexpr int kB = batch_slots<kSharedAlpha>();
  __shared__ int s_ent[kWaves][kRoundSlots];
  __shared__ float s_p[kWaves][kRoundSlots];
  const int w = threadIdx.x / kWave;
  const int seg = uniform(static_cast<int>(by * kWaves + w));
  if (seg >= part.nseg) return;
  const int lane = threadIdx.x % kWave;
  const int h0 = (bx * kWave + lane) * 8;
  const bool hin = h0 < H;
  const int c0 = bz * kConstGroup;
  const int64_t const_lo = int64_t(E) + sp.num_zero + sp.num_copy;
  const int64_t t_lo = int64_t(seg) * part.seg_len;
  const int64_t t_hi = t_lo + part.seg_len < T ? t_lo + part.seg_len : T;
  const int64_t s_hi = t_hi * K;

  float acv[kConstGroup][8], aa1[kConstGroup][8], aa2[kConstGroup][8];
#pragma unroll
  for (int q = 0; q < kConstGroup; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) acv[q][i] = aa1[q][i] = aa2[q][i] = 0.f;

  for (int64_t base = t_lo * K; base < s_hi; base += kRoundSlots) {
    // all 16 loads first (slots past the segment read its last slot instead)
    int idv[8];
    float pp[8];
    bool act[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t s = base + j * kWave + lane;
      const int64_t sl = s < s_hi ? s : s_hi - 1;
      idv[j] = ids[sl];
      pp[j] = probs[sl];
      act[j] = mk.active(sl);
    }
    int cq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = int64_t(idv[j]) - const_lo;
      const bool ok = base + j * kWave + lane < s_hi && act[j] && c >= c0 &&
                      c < c0 + kConstGroup && c < sp.num_const;
      cq[j] = ok ? static_cast<int>(c - c0) : -1;
    }
    int count = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool mine = cq[j] >= 0;
      const uint64_t m = ballot(mine);
      if (mine) {
        const int pos = count + rank_below(m);
        s_ent[w][pos] = ((j * kWave + lane) << 2) | cq[j];
        s_p[w][pos] = pp[j];
      }
      count += __builtin_popcountll(m);
    }
    __builtin_amdgcn_wave_barrier();
    for (int b = 0; b < count; b += kB) {
      // list entries past the end repeat entry b with no weight, so that every
      // load below is issued unconditionally and all are in flight together
      int jq[kB];
      float jp[kB];
      int64_t jt[kB];
      const int64_t seg_base = base - t_lo * K;  // slots of this segment before the round
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const bool ok = b + u < count;
        const int e = s_ent[w][ok ? b + u : b];
        const float pe = s_p[w][ok ? b + u : b];
        jq[u] = ok ? (e & 3) : -1;
        jp[u] = ok ? pe : 0.f;
        jt[u] = t_lo + static_cast<int64_t>(static_cast<uint32_t>(seg_base + (e >> 2)) /
                                            static_cast<uint32_t>(K));
      }
      const int hl = hin ? h0 : 0;
      float g[kB][8], al2[kB][8], x[kB][8], cv[kB][8];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t c = c0 + (jq[u] < 0 ? 0 : jq[u]);
        const int64_t abase = jt[u] * sp.a_st + c * sp.a_sc;
        unpack8(load16(grad_out + jt[u] * H + hl), g[u]);
        if (kSharedAlpha) {
          unpack8(load16(sp.ori_x + jt[u] * H + hl), x[u]);
          unpack8(load16(sp.const_v + c * H + hl), cv[u]);
        }
        if (kAlphaPerH) {
#pragma unroll
          for (int i = 0; i < 8; ++i) al2[u][i] = sp.alpha2[abase + int64_t(hl + i) * sp.a_sh];
        } else {
          const float a = sp.alpha2[abase];
#pragma unroll
          for (int i = 0; i < 8; ++i) al2[u][i] = a;
        }
      }
      if (hin) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
#pragma unroll
          for (int q = 0; q < kConstGroup; ++q) {
            if (jq[u] != q) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float pg = jp[u] * g[u][i];
              acv[q][i] = __builtin_fmaf(pg, al2[u][i], acv[q][i]);
              if (kSharedAlpha) {
                aa1[q][i] = __builtin_fmaf(pg, x[u][i], aa1[q][i]);
                aa2[q][i] = __builtin_fmaf(pg, cv[u][i], aa2[q][i]);
              }
            }
          }
        }
      }
    }
    // the list is rewritten by the next round only after every lane read it
    __builtin_amdgcn_wave_barrier();
  }
  if (!hin) return;
#pragma unroll
  for (int q = 0; q < kConstGroup; ++q) {
    const int c = c0 + q;
    if (c >= sp.num_const) break;
    const int64_t off = (int64_t(seg) * sp.num_const + c) * H + h0;
    float4* dst = reinterpret_cast<float4*>(part.cv + off);
    dst[0] = make_float4(acv[q][0], acv[q][1], acv[q][2], acv[q][3]);
    dst[1] = make_float4(acv[q][4], acv[q][5], acv[q][6], acv[q][7]);
    if (kSharedAlpha) {
      float4* d1 = reinterpret_cast<float4*>(part.a1 + off);
      d1[0] = make_float4(aa1[q][0], aa1[q][1], aa1[q][2], aa1[q][3]);
      d1[1] = make_float4(aa1[q][4], aa1[q][5], aa1[q][6], aa1[q][7]);
      float4* d2 = reinterpret_cast<float4*>(part.a2 + off);
      d2[0] = make_float4(aa2[q][0], aa2[q][1], aa2[q][2], aa2[q][3]);
      d2[1] = make_float4(aa2[q][4], aa2[q][5], aa2[q][6], aa2[q][7]);
    }
  }
}

template <bool kAlphaPerH, bool kSharedAlpha>
__global__ void __launch_bounds__(kWaves * kWave)
k_const_grad_partial(const uint16_t* __restrict__ grad_out, const int32_t* __restrict__ ids,
                     const float* __restrict__ probs, SlotMask mk, int64_t T, int K, int H, int E,
                     SpecialArgs sp, Partials part) {
  const_grad_partial_block<kAlphaPerH, kSharedAlpha>(
      static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z),
      grad_out, ids, probs, mk, T, K, H, E, sp, part);
}

// One launch, two roles, for the layout whose two bodies fit the same register
// budget (per-token alpha, K <= 8): the first n_part workgroups compute the
// const-expert partial sums (grid px x py x pz, flattened), the others the
// per-token gradients. The partial sums depend only on the inputs, so they
// run beside the per-token work instead of after it.
template <bool kHasRowMap>
__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(4)))
k_combine_grad_with_partials(const uint16_t* __restrict__ grad_out,
                             const uint16_t* __restrict__ expert_out, int64_t N,
                             const int32_t* __restrict__ row_of_slot,
                             const int32_t* __restrict__ row_map, const int32_t* __restrict__ ids,
                             const float* __restrict__ probs, SlotMask mk, int64_t T, int K,
                             int H, int E, SpecialArgs sp, CombineGradArgs o, int alpha_token,
                             int nsplit, Partials part, int px, int py, int n_part) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < n_part)
    const_grad_partial_block<false, false>(b % px, (b / px) % py, b / (px * py), grad_out, ids,
                                           probs, mk, T, K, H, E, sp, part);
  else
    combine_grad_tokens<kHasRowMap, false, 8>(b - n_part, grad_out, expert_out, N, row_of_slot,
                                              row_map, ids, probs, mk, T, K, H, E, sp, o,
                                              alpha_token, nsplit);
}

__device__ __forceinline__ void add4(float4& a, const float4& b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

// d_const_v[c,h] = bf16(sum over segments), and d_alpha[c*sc + h] for the
// shared layout that runs along h (stride_h == 1). A block covers 256
// consecutive (c, h) elements: lane l of each wave owns 4 of them, wave w
// adds segments w, w + 4, ... (four loads in flight), and the four waves'
// sums are added in LDS in wave order.
constexpr int kRedCols = kWave;          // float4 columns per block
__global__ void __launch_bounds__(kWaves * kWave)
k_const_grad_reduce(Partials part, int num_const, int H, int64_t a_sc, uint16_t* d_const_v,
                    float* d_alpha1, float* d_alpha2, int alpha_along_h) {
  __shared__ float4 red[3][kWaves][kRedCols];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t n_el = int64_t(num_const) * H;
  const int64_t e4 = (int64_t(blockIdx.x) * kRedCols + lane) * 4;
  const bool in = e4 < n_el;
  const bool want_alpha = alpha_along_h && (d_alpha1 != nullptr || d_alpha2 != nullptr);
  float4 scv = make_float4(0.f, 0.f, 0.f, 0.f), s1 = scv, s2 = scv;
  if (in) {
    int seg = w;
    for (; seg + 3 * kWaves < part.nseg; seg += 4 * kWaves) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = *reinterpret_cast<const float4*>(part.cv + int64_t(seg + u * kWaves) * n_el + e4);
#pragma unroll
      for (int u = 0; u < 4; ++u) add4(scv, v[u]);
      if (want_alpha) {
        float4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t off = int64_t(seg + u * kWaves) * n_el + e4;
          a[u] = *reinterpret_cast<const float4*>(part.a1 + off);
          b[u] = *reinterpret_cast<const float4*>(part.a2 + off);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          add4(s1, a[u]);
          add4(s2, b[u]);
        }
      }
    }
    for (; seg < part.nseg; seg += kWaves) {
      const int64_t off = int64_t(seg) * n_el + e4;
      add4(scv, *reinterpret_cast<const float4*>(part.cv + off));
      if (want_alpha) {
        add4(s1, *reinterpret_cast<const float4*>(part.a1 + off));
        add4(s2, *reinterpret_cast<const float4*>(part.a2 + off));
      }
    }
  }
  red[0][w][lane] = scv;
  red[1][w][lane] = s1;
  red[2][w][lane] = s2;
  __syncthreads();
  if (w != 0 || !in) return;
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    add4(scv, red[0][i][lane]);
    add4(s1, red[1][i][lane]);
    add4(s2, red[2][i][lane]);
  }
  if (d_const_v != nullptr) {
    const uint2 packed = make_uint2(pack_bf16x2(scv.x, scv.y), pack_bf16x2(scv.z, scv.w));
    *reinterpret_cast<uint2*>(d_const_v + e4) = packed;
  }
  if (want_alpha) {
    const int c = static_cast<int>(e4 / H);
    const int h = static_cast<int>(e4 % H);
    const int64_t ai = int64_t(c) * a_sc + h;
    const float r1[4] = {s1.x, s1.y, s1.z, s1.w}, r2[4] = {s2.x, s2.y, s2.z, s2.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (d_alpha1 != nullptr) d_alpha1[ai + i] = r1[i];
      if (d_alpha2 != nullptr) d_alpha2[ai + i] = r2[i];
    }
  }
}

// Shared layouts that do not run along h (stride_h == 0): one block per
// alpha element (c*sc, or the single element when sc == 0), summing the
// partials over segments, h (and c when sc == 0).
__global__ void __launch_bounds__(256)
k_alpha_grad_reduce(Partials part, int num_const, int H, int64_t a_sc, float* d_alpha1,
                    float* d_alpha2) {
  __shared__ float red[2][256 / kWave];
  const int el = blockIdx.x;
  const int c_lo = a_sc == 0 ? 0 : el, c_hi = a_sc == 0 ? num_const : el + 1;
  float v1 = 0.f, v2 = 0.f;
  for (int seg = 0; seg < part.nseg; ++seg)
    for (int c = c_lo; c < c_hi; ++c) {
      const int64_t base = (int64_t(seg) * num_const + c) * H;
      for (int h = threadIdx.x; h < H; h += blockDim.x) {
        v1 += part.a1[base + h];
        v2 += part.a2[base + h];
      }
    }
  v1 = wave_sum(v1);
  v2 = wave_sum(v2);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    red[0][w] = v1;
    red[1][w] = v2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float r1 = 0.f, r2 = 0.f;
    for (int i = 0; i < static_cast<int>(blockDim.x) / kWave; ++i) {
      r1 += red[0][i];
      r2 += red[1][i];
    }
    const int64_t ai = int64_t(el) * a_sc;
    if (d_alpha1 != nullptr) d_alpha1[ai] = r1;
    if (d_alpha2 != nullptr) d_alpha2[ai] = r2;
  }
}

struct SegPlan {
  int nseg;
  int64_t seg_len;
};

// Token segments of the partial sums: about one round (512 slots) each, at
// most kMaxSegments of them.
SegPlan seg_plan(int64_t T, int K) {
  const int64_t t = T > 0 ? T : 1;
  int64_t nseg = ceil_div(t * K, kRoundSlots);
  if (nseg > kMaxSegments) nseg = kMaxSegments;
  if (nseg < 1) nseg = 1;
  const int64_t len = ceil_div(t, nseg);
  return SegPlan{static_cast<int>(ceil_div(t, len)), len};
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

AlphaLayout classify_alpha(const SpecialArgs& sp, int H) {
  if (sp.num_const <= 0) return AlphaLayout::kNone;
  const int64_t st = sp.a_st, sc = sp.a_sc, sh = sp.a_sh;
  if (st < 0 || sc < 0 || sh < 0) return AlphaLayout::kOther;
  if (st > 0 && sh == 0 && int64_t(sp.num_const - 1) * sc < st) return AlphaLayout::kPerToken;
  if (st == 0 && sh == 0) return AlphaLayout::kSharedScalar;
  if (st == 0 && sh == 1 && (sc >= H || sp.num_const == 1)) return AlphaLayout::kSharedAlongH;
  return AlphaLayout::kOther;
}

size_t combine_grad_workspace_bytes(int64_t T, int H, int num_const) {
  if (num_const <= 0) return 256;
  const SegPlan sg = seg_plan(T, 16);  // the most segments any K <= 16 uses
  return 3 * align256(size_t(sg.nseg) * size_t(num_const) * size_t(H) * sizeof(float));
}

hipError_t launch_combine_grad(const uint16_t* grad_out, const uint16_t* expert_out, int64_t N,
                               const int32_t* row_of_slot, const int32_t* row_map,
                               const int32_t* ids, const float* probs, SlotMask mk, int64_t T,
                               int K, int H, int E, const SpecialArgs& sp,
                               const CombineGradArgs& o, void* ws, hipStream_t st) {
  if (T == 0) return hipGetLastError();
  const AlphaLayout lay = classify_alpha(sp, H);
  const bool want_alpha = o.d_alpha1 != nullptr || o.d_alpha2 != nullptr;
  const bool per_h = sp.num_const > 0 && sp.a_sh != 0;
  const int alpha_token = want_alpha && lay == AlphaLayout::kPerToken;
  const bool shared_alpha =
      want_alpha && (lay == AlphaLayout::kSharedAlongH || lay == AlphaLayout::kSharedScalar);
  const bool need_part = sp.num_const > 0 && (o.d_const_v != nullptr || shared_alpha);
  // four (or two) waves per token once a token's row is long and there are
  // too few tokens to keep every SIMD busy for several rounds
  const int nsplit = T >= 2 * kSplitBelowTokens ? 1
                     : H / 8 >= 4 * kWave       ? 4
                     : H / 8 >= 2 * kWave       ? 2
                                                : 1;
  const int64_t main_blocks = ceil_div(T, kWaves / nsplit);
  const dim3 block(kWaves * kWave);
  Partials part{};
  int px = 0, py = 0, pz = 0;
  if (need_part) {
    const SegPlan sg = seg_plan(T, K);
    const size_t slab =
        align256(size_t(sg.nseg) * size_t(sp.num_const) * size_t(H) * sizeof(float));
    char* base = static_cast<char*>(ws);
    part = Partials{reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + slab),
                    reinterpret_cast<float*>(base + 2 * slab), sg.nseg, sg.seg_len};
    px = static_cast<int>(ceil_div(H, kTileH));
    py = static_cast<int>(ceil_div(sg.nseg, kWaves));
    pz = static_cast<int>(ceil_div(sp.num_const, kConstGroup));
  }
  if (need_part && !per_h && !shared_alpha && K <= 8) {
    // the partial sums and the per-token work in one launch
    const int n_part = px * py * pz;
    const dim3 grid(static_cast<unsigned>(n_part + main_blocks));
    if (row_map != nullptr)
      hipLaunchKernelGGL(k_combine_grad_with_partials<true>, grid, block, 0, st, grad_out,
                         expert_out, N, row_of_slot, row_map, ids, probs, mk, T, K, H, E, sp, o,
                         alpha_token, nsplit, part, px, py, n_part);
    else
      hipLaunchKernelGGL(k_combine_grad_with_partials<false>, grid, block, 0, st, grad_out,
                         expert_out, N, row_of_slot, row_map, ids, probs, mk, T, K, H, E, sp, o,
                         alpha_token, nsplit, part, px, py, n_part);
  } else {
    const dim3 grid(static_cast<unsigned>(main_blocks));
#define MOE_CGRAD(RM, PH, MK)                                                                    hipLaunchKernelGGL((k_combine_grad<RM, PH, MK>), grid, block, 0, st, grad_out, expert_out, N,                      row_of_slot, row_map, ids, probs, mk, T, K, H, E, sp, o, alpha_token,                         nsplit)
#define MOE_CGRAD_K(RM, PH) \
  if (K <= 8) MOE_CGRAD(RM, PH, 8); else MOE_CGRAD(RM, PH, 16);
    if (row_map != nullptr) {
      if (per_h) { MOE_CGRAD_K(true, true) } else { MOE_CGRAD_K(true, false) }
    } else {
      if (per_h) { MOE_CGRAD_K(false, true) } else { MOE_CGRAD_K(false, false) }
    }
#undef MOE_CGRAD_K
#undef MOE_CGRAD
    if (need_part) {
      const dim3 pgrid(static_cast<unsigned>(px), static_cast<unsigned>(py),
                       static_cast<unsigned>(pz));
#define MOE_CPART(PH, SA)                                                                   \
  hipLaunchKernelGGL((k_const_grad_partial<PH, SA>), pgrid, block, 0, st, grad_out, ids, probs, \
                     mk, T, K, H, E, sp, part)
      if (per_h) {
        if (shared_alpha) MOE_CPART(true, true); else MOE_CPART(true, false);
      } else {
        if (shared_alpha) MOE_CPART(false, true); else MOE_CPART(false, false);
      }
#undef MOE_CPART
    }
  }
  if (!need_part) return hipGetLastError();

  const int64_t n4 = int64_t(sp.num_const) * H / 4;
  hipLaunchKernelGGL(k_const_grad_reduce, dim3(static_cast<unsigned>(ceil_div(n4, kRedCols))),
                     dim3(kWaves * kWave), 0, st, part, sp.num_const, H, sp.a_sc, o.d_const_v,
                     shared_alpha ? o.d_alpha1 : nullptr, shared_alpha ? o.d_alpha2 : nullptr,
                     shared_alpha && lay == AlphaLayout::kSharedAlongH ? 1 : 0);
  if (shared_alpha && lay == AlphaLayout::kSharedScalar) {
    const int n_el = sp.a_sc == 0 ? 1 : sp.num_const;
    hipLaunchKernelGGL(k_alpha_grad_reduce, dim3(static_cast<unsigned>(n_el)), dim3(256), 0, st,
                       part, sp.num_const, H, sp.a_sc, o.d_alpha1, o.d_alpha2);
  }
  return hipGetLastError();
}

}  // namespace moe
