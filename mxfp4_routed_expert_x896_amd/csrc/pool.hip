// Expert pool: keeps the records of the experts a call routes to resident in
// a fixed set of HBM slots, copying the missing ones from host memory.
//
// Deltafin README, I/O and streaming: the experts are read from storage as
// whole contiguous records when the router selects them, and the records of
// recent tokens are kept; Deltafin explainer, section 6.1: the I/O path, not
// the arithmetic, decides the speed once the model exceeds memory.  Here the
// storage is pinned host memory, each record one host-to-device DMA copy,
// and the pool evicts the slot used longest ago among the experts the call
// does not need.  The bookkeeping is host-side; the device sees the records
// in their slots and the slot map the layer kernels read (expert_slot).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe_mxfp4.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

struct moe_expert_pool {
  const uint8_t* host;  // E packed records, stride apart (host)
  uint64_t stride;
  int32_t n_experts;
  uint8_t* slots;       // n_slots records, stride apart (device)
  int32_t n_slots;
  int32_t* slot_map;    // [E] (device)
  std::vector<int32_t> slot_of;   // expert -> slot, -1 if not resident
  std::vector<int32_t> owner;     // slot -> expert, -1 if free
  std::vector<uint64_t> used_at;  // slot -> fetch counter of its last use
  uint64_t clock = 0;
  int64_t copied = 0, resident = 0;
};

namespace {

// Slot-map entries written by one launch (kernel arguments, so nothing on
// the host has to outlive the call).
constexpr int kMapBatch = 32;
struct MapUpdate {
  int32_t expert[kMapBatch];
  int32_t slot[kMapBatch];
  int32_t n;
};

__global__ void pool_map_fill(int32_t* map, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) map[i] = 0;
}

__global__ void pool_map_update(int32_t* map, MapUpdate u) {
  const int i = threadIdx.x;
  if (i < u.n) map[u.expert[i]] = u.slot[i];
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// After a failed copy or launch the slots' contents are unknown: forget
// every resident record, so later fetches copy what they need again.
int pool_failed(moe_expert_pool* p) {
  p->slot_of.assign(p->n_experts, -1);
  p->owner.assign(p->n_slots, -1);
  p->used_at.assign(p->n_slots, 0);
  return MOE_ELAUNCH;
}

}  // namespace

MOE_API int moe_pool_create(const uint8_t* host_records, uint64_t stride, int32_t n_experts,
                            uint8_t* slots, int32_t n_slots, int32_t* slot_map,
                            hipStream_t stream, moe_expert_pool** out_pool) {
  if (out_pool == nullptr) return MOE_EINVAL;
  *out_pool = nullptr;
  if (host_records == nullptr || slots == nullptr || slot_map == nullptr || stride == 0 ||
      n_experts <= 0 || n_slots <= 0)
    return MOE_EINVAL;
  if (n_slots > n_experts || n_experts > 1024) return MOE_ESHAPE;
  if ((stride & 15u) || !aligned(slots, 16) || !aligned(slot_map, 4)) return MOE_EALIGN;
  moe_expert_pool* p = new (std::nothrow) moe_expert_pool();
  if (p == nullptr) return MOE_ELAUNCH;
  p->host = host_records;
  p->stride = stride;
  p->n_experts = n_experts;
  p->slots = slots;
  p->n_slots = n_slots;
  p->slot_map = slot_map;
  p->slot_of.assign(n_experts, -1);
  p->owner.assign(n_slots, -1);
  p->used_at.assign(n_slots, 0);
  hipLaunchKernelGGL(pool_map_fill, dim3((n_experts + 255) / 256), dim3(256), 0, stream,
                     slot_map, n_experts);
  if (hipGetLastError() != hipSuccess) {
    delete p;
    return MOE_ELAUNCH;
  }
  *out_pool = p;
  return MOE_OK;
}

MOE_API int moe_pool_fetch(moe_expert_pool* p, const int32_t* ids, int64_t n_ids,
                           hipStream_t stream, int32_t* copied) {
  if (copied != nullptr) *copied = 0;
  if (p == nullptr || ids == nullptr || n_ids <= 0) return MOE_EINVAL;
  for (int64_t i = 0; i < n_ids; ++i)
    if (ids[i] < 0 || ids[i] >= p->n_experts) return MOE_EINVAL;
  // the distinct experts of this call, in first-seen order
  std::vector<char> need(p->n_experts, 0);
  std::vector<int32_t> want;
  for (int64_t i = 0; i < n_ids; ++i)
    if (!need[ids[i]]) {
      need[ids[i]] = 1;
      want.push_back(ids[i]);
    }
  if (int64_t(want.size()) > p->n_slots) return MOE_ESHAPE;
  const uint64_t now = ++p->clock;
  std::vector<int32_t> missing;
  for (int32_t e : want) {
    if (p->slot_of[e] >= 0) {
      p->used_at[p->slot_of[e]] = now;
      ++p->resident;
    } else {
      missing.push_back(e);
    }
  }
  MapUpdate u;
  u.n = 0;
  int n_copied = 0;
  for (int32_t e : missing) {
    // a free slot, else the least recently used one whose expert this call
    // does not need (there is one: at most n_slots experts are needed, and
    // the needed resident ones were just stamped with `now`)
    int victim = -1;
    for (int s = 0; s < p->n_slots && victim < 0; ++s)
      if (p->owner[s] < 0) victim = s;
    if (victim < 0) {
      uint64_t oldest = UINT64_MAX;
      for (int s = 0; s < p->n_slots; ++s)
        if (p->used_at[s] < now && !need[p->owner[s]] && p->used_at[s] < oldest) {
          oldest = p->used_at[s];
          victim = s;
        }
    }
    if (victim < 0) return pool_failed(p);  // unreachable given the size check
    if (p->owner[victim] >= 0) p->slot_of[p->owner[victim]] = -1;
    if (hipMemcpyAsync(p->slots + uint64_t(victim) * p->stride, p->host + uint64_t(e) * p->stride,
                       p->stride, hipMemcpyHostToDevice, stream) != hipSuccess)
      return pool_failed(p);
    p->owner[victim] = e;
    p->slot_of[e] = victim;
    p->used_at[victim] = now;
    ++n_copied;
    u.expert[u.n] = e;
    u.slot[u.n] = victim;
    if (++u.n == kMapBatch) {
      hipLaunchKernelGGL(pool_map_update, dim3(1), dim3(kMapBatch), 0, stream, p->slot_map, u);
      if (hipGetLastError() != hipSuccess) return pool_failed(p);
      u.n = 0;
    }
  }
  if (u.n > 0) {
    hipLaunchKernelGGL(pool_map_update, dim3(1), dim3(kMapBatch), 0, stream, p->slot_map, u);
    if (hipGetLastError() != hipSuccess) return pool_failed(p);
  }
  p->copied += n_copied;
  if (copied != nullptr) *copied = n_copied;
  return MOE_OK;
}

MOE_API int moe_pool_stats(const moe_expert_pool* p, int64_t* copied, int64_t* resident) {
  if (p == nullptr) return MOE_EINVAL;
  if (copied != nullptr) *copied = p->copied;
  if (resident != nullptr) *resident = p->resident;
  return MOE_OK;
}

MOE_API int moe_pool_destroy(moe_expert_pool* p) {
  if (p == nullptr) return MOE_EINVAL;
  delete p;
  return MOE_OK;
}
