// Exported C entry points of libmxmoe.so: argument checks, device check,
// error reporting, enum names.  Every check runs before the first enqueue.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace mxmoe {

static thread_local std::string g_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

void clear_error() { g_error.clear(); }

namespace {
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;    // -1 unknown, 0 no, 1 yes
std::vector<int> g_dev_cus;

int device_index(int* dev) { return hipGetDevice(dev) == hipSuccess ? 0 : -1; }

moe_status query_device(int dev) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev_ok.size() <= dev) {
    g_dev_ok.resize(dev + 1, -1);
    g_dev_cus.resize(dev + 1, 0);
  }
  if (g_dev_ok[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipGetDeviceProperties(%d) failed", dev);
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    g_dev_cus[dev] = prop.multiProcessorCount;
    if (!g_dev_ok[dev])
      return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library runs on gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (!g_dev_ok[dev]) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d is not a gfx950", dev);
  return MOE_OK;
}
}  // namespace

moe_status check_device() {
  int dev = 0;
  if (device_index(&dev) != 0) return fail(MOE_ERR_HIP, "hipGetDevice failed (no HIP device?)");
  return query_device(dev);
}

int num_cus() {
  int dev = 0;
  if (device_index(&dev) != 0) return 256;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return dev < (int)g_dev_cus.size() && g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256;
}

}  // namespace mxmoe

using namespace mxmoe;

extern "C" {

int moe_abi_version(void) { return MXMOE_ABI_VERSION; }

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE";
    case MOE_ERR_NOT_PINNED: return "MOE_ERR_NOT_PINNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_NOT_IMPLEMENTED: return "MOE_ERR_NOT_IMPLEMENTED";
    default: return "unknown status";
  }
}

const char* moe_last_error_message(void) { return g_error.c_str(); }

const char* moe_enum_name(int kind, int v) {
  switch (kind) {
    case MOE_ENUM_STATUS: return (v >= 0 && v <= 7) ? moe_status_string(v) : nullptr;
    case MOE_ENUM_ACT:
      return v == MOE_ACT_BF16 ? "MOE_ACT_BF16" : v == MOE_ACT_MXFP8_E4M3 ? "MOE_ACT_MXFP8_E4M3" : nullptr;
    case MOE_ENUM_OUT:
      return v == MOE_OUT_FP32 ? "MOE_OUT_FP32"
             : v == MOE_OUT_BF16 ? "MOE_OUT_BF16"
             : v == MOE_OUT_MXFP8_E4M3 ? "MOE_OUT_MXFP8_E4M3" : nullptr;
    case MOE_ENUM_EPI:
      return v == MOE_EPI_NONE ? "MOE_EPI_NONE"
             : v == MOE_EPI_SWIGLU_SPLIT ? "MOE_EPI_SWIGLU_SPLIT"
             : v == MOE_EPI_SWIGLU_INTERLEAVED ? "MOE_EPI_SWIGLU_INTERLEAVED" : nullptr;
    case MOE_ENUM_CHAIN:
      return v == MOE_CHAIN_RMS ? "MOE_CHAIN_RMS" : v == MOE_CHAIN_INDEPENDENT ? "MOE_CHAIN_INDEPENDENT" : nullptr;
    case MOE_ENUM_WFORMAT:
      return v == MOE_W_CANONICAL ? "MOE_W_CANONICAL" : v == MOE_W_TILED ? "MOE_W_TILED" : nullptr;
    case MOE_ENUM_COPY:
      return v == MOE_COPY_ALL ? "MOE_COPY_ALL"
             : v == MOE_COPY_ROUTED ? "MOE_COPY_ROUTED"
             : v == MOE_COPY_AUTO ? "MOE_COPY_AUTO" : nullptr;
    default: return nullptr;
  }
}

int moe_device_supported(void) {
  clear_error();
  moe_status s = check_device();
  return s == MOE_OK ? 1 : s == MOE_ERR_UNSUPPORTED_DEVICE ? 0 : -1;
}

moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_w, void* stream) {
  clear_error();
  if (T < 0) return fail(MOE_ERR_SHAPE, "route: T = %d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "route: E = %d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 64) return fail(MOE_ERR_SHAPE, "route: k = %d outside [1, min(E=%d, 64)]", k, E);
  if (T > 0 && (!logits || !topk_ids || !topk_w)) return fail(MOE_ERR_INVALID_ARG, "route: null pointer");
  MXMOE_TRY(check_device());
  return launch_route(logits, T, E, k, topk_ids, topk_w, (hipStream_t)stream);
}

size_t moe_permute_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return permute_ws_bytes(T, E, k);
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k, int32_t* expert_offsets,
                       int32_t* perm_src, int32_t* dest_row, void* workspace, size_t workspace_bytes,
                       void* stream) {
  clear_error();
  if (T < 0) return fail(MOE_ERR_SHAPE, "permute: T = %d < 0", T);
  if (E < 1 || E > 8192) return fail(MOE_ERR_SHAPE, "permute: E = %d outside [1, 8192]", E);
  if (k < 1 || k > E) return fail(MOE_ERR_SHAPE, "permute: k = %d outside [1, E=%d]", k, E);
  if ((int64_t)T * k >= (1ll << 31)) return fail(MOE_ERR_SHAPE, "permute: T*k overflows int32");
  if (!expert_offsets || (T > 0 && (!topk_ids || !perm_src || !dest_row)))
    return fail(MOE_ERR_INVALID_ARG, "permute: null pointer");
  const size_t need = permute_ws_bytes(T, E, k);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "permute: workspace %zu bytes, need %zu", workspace_bytes, need);
  MXMOE_TRY(check_device());
  return launch_permute(topk_ids, T, E, k, expert_offsets, perm_src, dest_row, workspace,
                        (hipStream_t)stream);
}

size_t moe_grouped_gemm_workspace_size(const moe_gemm_args* a) {
  if (!a || a->rows < 0 || a->E < 1) return 0;
  return gemm_ws_bytes(a->rows, a->E);
}

moe_status moe_mxfp4_grouped_gemm(const moe_gemm_args* a, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  clear_error();
  if (!a) return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: null args");
  MXMOE_TRY(validate_gemm(*a));
  const size_t need = gemm_ws_bytes(a->rows, a->E);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "grouped GEMM: workspace %zu bytes, need %zu", workspace_bytes, need);
  MXMOE_TRY(check_device());
  return launch_gemm(*a, workspace, (hipStream_t)stream);
}

size_t moe_tiled_weight_bytes(int32_t E, int32_t N, int32_t K, int32_t which) { return tiled_bytes(E, N, K, which); }

static moe_status tile_common(const uint8_t* sp, const uint8_t* ss, int32_t E, int32_t N, int32_t K, int32_t epi,
                              uint8_t* dp, uint8_t* ds, bool to_tiled, void* stream) {
  const char* what = to_tiled ? "tile weights" : "untile weights";
  if (!tile_shape_ok(E, N, K))
    return fail(MOE_ERR_SHAPE, "%s: needs E >= 1, K %% 512 == 0 and N %% 256 == 0 (E %d, N %d, K %d)", what, E, N, K);
  if (epi < MOE_EPI_NONE || epi > MOE_EPI_SWIGLU_INTERLEAVED)
    return fail(MOE_ERR_INVALID_ARG, "%s: bad epilogue %d", what, epi);
  if (!sp || !ss || !dp || !ds) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
  const size_t bp = tiled_bytes(E, N, K, 0), bs = tiled_bytes(E, N, K, 1);
  auto overlap = [](const uint8_t* a, size_t na, const uint8_t* b, size_t nb) { return a < b + nb && b < a + na; };
  if (overlap(sp, bp, dp, bp) || overlap(sp, bp, ds, bs) || overlap(ss, bs, dp, bp) || overlap(ss, bs, ds, bs))
    return fail(MOE_ERR_INVALID_ARG, "%s: input and output overlap", what);
  MXMOE_TRY(check_device());
  return launch_tile(sp, ss, E, N, K, epi, dp, ds, to_tiled, (hipStream_t)stream);
}

moe_status moe_mxfp4_tile_weights(const uint8_t* w_packed, const uint8_t* w_scales, int32_t E, int32_t N, int32_t K,
                                  int32_t epilogue, uint8_t* t_packed, uint8_t* t_scales, void* stream) {
  clear_error();
  return tile_common(w_packed, w_scales, E, N, K, epilogue, t_packed, t_scales, true, stream);
}

moe_status moe_mxfp4_untile_weights(const uint8_t* t_packed, const uint8_t* t_scales, int32_t E, int32_t N,
                                    int32_t K, int32_t epilogue, uint8_t* w_packed, uint8_t* w_scales, void* stream) {
  clear_error();
  return tile_common(t_packed, t_scales, E, N, K, epilogue, w_packed, w_scales, false, stream);
}

moe_status moe_combine(const void* y, int32_t y_dtype, const int32_t* dest_row, const float* topk_w,
                       int32_t T, int32_t k, int32_t H, float* out, uint16_t* x_next, void* stream) {
  clear_error();
  if (y_dtype != MOE_OUT_FP32 && y_dtype != MOE_OUT_BF16)
    return fail(MOE_ERR_INVALID_ARG, "combine: y_dtype %d must be MOE_OUT_FP32 or MOE_OUT_BF16", y_dtype);
  if (T < 0 || k < 1 || H < 1) return fail(MOE_ERR_SHAPE, "combine: T %d, k %d, H %d out of range", T, k, H);
  if (H % 8) return fail(MOE_ERR_SHAPE, "combine: H = %d must be a multiple of 8", H);
  if (T > 0 && (!y || !dest_row || !topk_w || !out)) return fail(MOE_ERR_INVALID_ARG, "combine: null pointer");
  MXMOE_TRY(check_device());
  return launch_combine(y, y_dtype, dest_row, topk_w, T, k, H, out, x_next, (hipStream_t)stream);
}

}  // extern "C"
