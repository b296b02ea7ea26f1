// The grouped GEMM for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// moe_mxfp4_grouped_gemm takes its planner scratch (per-class tile lists, tile
// counts and per-XCD unit counters) from a caller workspace.  This variant
// takes it from `scratch`, a file-scope device array of a fixed size that
// every device the library runs on holds for the life of the process.  The
// kernels are the same ones; they receive the array's device address as their
// workspace argument, looked up once per device with hipGetSymbolAddress (in
// host code the array's name is only a host-side stand-in, never a device
// address).  The planner kernel writes every word the GEMM kernels read
// (lists, counts) and zeroes the unit counters itself, so a call needs no
// clearing and leaves nothing a later call depends on.
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kStaticScratchBytes = MXMOE_STATIC_SCRATCH_BYTES;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace mxmoe {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)

// The current device's copy of `scratch`, looked up on that device's first call.
moe_status device_scratch(void** out) {
  int dev = 0;
  MXMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED_DEVICE, "grouped GEMM (static scratch): device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    MXMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(MOE_ERR_HIP, "grouped GEMM (static scratch): no device address for the scratch array");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace mxmoe

using namespace mxmoe;

extern "C" {

moe_status moe_mxfp4_grouped_gemm_static(const moe_gemm_args* a, void* stream) {
  clear_error();
  if (!a) return fail(MOE_ERR_INVALID_ARG, "grouped GEMM (static scratch): null args");
  MXMOE_TRY(validate_gemm(*a));
  const size_t need = gemm_ws_bytes(a->rows, a->E);
  if (need > kStaticScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "grouped GEMM (static scratch): rows %d and E %d need %zu bytes of scratch, the static array "
                "holds %zu (use moe_mxfp4_grouped_gemm with a workspace)",
                a->rows, a->E, need, kStaticScratchBytes);
  MXMOE_TRY(check_device());
  void* ws = nullptr;
  MXMOE_TRY(device_scratch(&ws));
  return launch_gemm(*a, ws, (hipStream_t)stream);
}

}  // extern "C"
