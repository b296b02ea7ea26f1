// Routed expert copy for the streamed prefill: moves, from a layer's
// page-locked host blob into its HBM slot, only the experts that received at
// least one routed row of this layer (the routing-aware variant of the
// layerwise expert stream, ktransformers issue #2172: the serialized chain
// loads all experts of a layer, "Impact"; the experts a batch does not hit
// need not cross the host link).
//
// The set of hit experts is known only on the device (expert_offsets of the
// layer's permutation), so the copy is a kernel that reads the device-mapped
// host blob over the host link, not a copy-engine transfer whose sizes the
// host would have to know.  Each expert occupies one contiguous byte range
// per blob section, in the canonical and in the tiled weight order alike.
#include "internal.h"

namespace mxmoe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 1024;   // 16 waves: one block fills one free CU
constexpr int kCopyLoads = 8;        // 16-byte loads in flight per thread
constexpr uint64_t kChunk = (uint64_t)kCopyThreads * kCopyLoads * 16;  // 128 KiB per unit

struct CopyPlan {
  const uint8_t* src[4];   // device-visible address of each host section
  uint8_t* dst[4];         // slot section
  uint64_t per_expert[4];  // bytes of one expert in each section, multiples of 16
  int chunks[4];           // units of one expert in each section
  int units_per_expert;
};

// Unit u = (expert u / units_per_expert, then section-major chunks).  A unit of
// an expert with no routed row is skipped by the whole block.
__global__ __launch_bounds__(kCopyThreads) void routed_copy_kernel(CopyPlan p, const int32_t* __restrict__ off,
                                                                  int E) {
  const int64_t units = (int64_t)E * p.units_per_expert;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int e = (int)(u / p.units_per_expert);
    if (off[e + 1] == off[e]) continue;
    int c = (int)(u % p.units_per_expert);
    int s = 0;
    if (c >= p.chunks[0]) { c -= p.chunks[0]; s = 1;
      if (c >= p.chunks[1]) { c -= p.chunks[1]; s = 2;
        if (c >= p.chunks[2]) { c -= p.chunks[2]; s = 3; } } }
    const uint64_t per = s == 0 ? p.per_expert[0] : s == 1 ? p.per_expert[1] : s == 2 ? p.per_expert[2] : p.per_expert[3];
    const uint8_t* sb = s == 0 ? p.src[0] : s == 1 ? p.src[1] : s == 2 ? p.src[2] : p.src[3];
    uint8_t* db = s == 0 ? p.dst[0] : s == 1 ? p.dst[1] : s == 2 ? p.dst[2] : p.dst[3];
    const uint64_t first = (uint64_t)c * kChunk;
    const uint64_t n16 = (min(per, first + kChunk) - first) / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(sb + (uint64_t)e * per + first);
    u32x4* dst = reinterpret_cast<u32x4*>(db + (uint64_t)e * per + first);
    u32x4 v[kCopyLoads];
#pragma unroll
    for (int i = 0; i < kCopyLoads; ++i) {
      const uint64_t j = (uint64_t)i * kCopyThreads + threadIdx.x;
      if (j < n16) v[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < kCopyLoads; ++i) {
      const uint64_t j = (uint64_t)i * kCopyThreads + threadIdx.x;
      if (j < n16) __builtin_nontemporal_store(v[i], dst + j);
    }
  }
}

}  // namespace

moe_status launch_routed_copy(const uint8_t* const src[4], uint8_t* const dst[4], const uint64_t per_expert[4],
                              const int32_t* expert_offsets, int E, int blocks, hipStream_t s) {
  CopyPlan p{};
  p.units_per_expert = 0;
  for (int i = 0; i < 4; ++i) {
    p.src[i] = src[i];
    p.dst[i] = dst[i];
    p.per_expert[i] = per_expert[i];
    p.chunks[i] = (int)((per_expert[i] + kChunk - 1) / kChunk);
    p.units_per_expert += p.chunks[i];
  }
  hipLaunchKernelGGL(routed_copy_kernel, dim3(blocks), dim3(kCopyThreads), 0, s, p, expert_offsets, E);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace mxmoe
