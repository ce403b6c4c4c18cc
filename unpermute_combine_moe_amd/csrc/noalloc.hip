// moe_permute_noalloc: moe_permute with its (chunk, expert) count table kept in
// a device array owned by the library instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// Every call on one GPU uses that GPU's copy of the array. Nothing in it has to
// start at zero: the count kernel of a call writes every table entry the same
// call reads afterwards. Two calls that overlap in time on one GPU (different
// streams) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "libmoeperm.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

// The largest count table the permute's planner makes: at most 16,384 int32
// entries for every legal T, K and E.
constexpr size_t kScratchBytes = 16384 * sizeof(int32_t);

// Host code must not pass `scratch` itself to a kernel (in host code it names a
// host-side stand-in); it uses the device address looked up below.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device

// Device address of `scratch` on the device `stream` belongs to, looked up
// once per device with that device current.
hipError_t scratch_for(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = (stream == nullptr) ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

MOE_API moe_status_t moe_permute_noalloc(const void* x, const int32_t* expert_ids,
                                         const uint8_t* active_mask, int32_t mask_per_slot,
                                         int64_t T, int32_t H, int32_t K, int32_t num_experts,
                                         void* permuted, int32_t* sorted_slot,
                                         int32_t* row_of_slot, int32_t* expert_counts,
                                         int32_t* expert_offsets, hipStream_t stream) {
  // the size check first, so that an oversized request fails before any HIP call
  size_t need = 0;
  if (moe_status_t s = moe_permute_workspace_size(T, K, num_experts, &need)) return s;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_for(stream, &ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_permute(x, expert_ids, active_mask, mask_per_slot, T, H, K, num_experts, permuted,
                     sorted_slot, row_of_slot, expert_counts, expert_offsets, ws, kScratchBytes,
                     stream);
}
