// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "mxmoe.h"

namespace mxmoe {

// ---- errors -----------------------------------------------------------
moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define MXMOE_HIP(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess)                                                            \
      return ::mxmoe::fail(MOE_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define MXMOE_TRY(expr)               \
  do {                                \
    moe_status s_ = (expr);           \
    if (s_ != MOE_OK) return s_;      \
  } while (0)

// Current device must be a gfx950; cached per device id.
moe_status check_device();
// Compute units of the current device (cached).
int num_cus();

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- launchers (arguments already validated) --------------------------
moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);
size_t permute_ws_bytes(int T, int E, int k);
moe_status launch_permute(const int32_t* ids, int T, int E, int k, int32_t* off, int32_t* perm_src,
                          int32_t* dest_row, void* ws, hipStream_t s);
size_t gemm_ws_bytes(int rows, int E);
// reserve: CUs per XCD that the persistent GEMM launches leave free (0: none).
// max_rows: a bound on any expert's row count (-1: the call's rows); row-tile
// classes no expert can fill are not launched.
moe_status launch_gemm(const moe_gemm_args& a, void* ws, hipStream_t s, int reserve = 0, int max_rows = -1);
moe_status launch_combine(const void* y, int y_dtype, const int32_t* dest_row, const float* w,
                          int T, int k, int H, float* out, uint16_t* x_next, hipStream_t s);
moe_status validate_gemm(const moe_gemm_args& a);
// routed expert copy (expert_copy.hip): copies expert e's byte range of each of
// the four sections when expert_offsets[e + 1] > expert_offsets[e]; `blocks`
// blocks of 1024 threads
moe_status launch_routed_copy(const uint8_t* const src[4], uint8_t* const dst[4], const uint64_t per_expert[4],
                              const int32_t* expert_offsets, int E, int blocks, hipStream_t s);
// load-time weight tiling (gemm.hip)
bool tile_shape_ok(int E, int N, int K);
size_t tiled_bytes(int E, int N, int K, int which);
moe_status launch_tile(const uint8_t* src_p, const uint8_t* src_s, int E, int N, int K, int layout,
                       uint8_t* dst_p, uint8_t* dst_s, bool to_tiled, hipStream_t s);

// ---- layer workspace layout -------------------------------------------
struct LayerWs {
  size_t ids, w, off, perm_src, dest_row, inter, inter_scales, y, permute_ws, gemm_ws, total;
};
LayerWs layer_ws_layout(int T, int H, int I, int E, int k, int inter_dtype);

}  // namespace mxmoe
