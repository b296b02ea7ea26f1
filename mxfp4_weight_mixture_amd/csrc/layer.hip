// One resident MoE layer, and the layerwise double-buffered streamed
// prefill over stacked layers.
//
// The streamed pass replaces the per-layer chain "H2D-load all experts ->
// compute -> hard sync -> next layer" (ktransformers issue #2172, "Impact")
// by the double-buffered layerwise pipeline the same issue asks for
// ("Background / motivation"): while layer L computes out of HBM slot L%2,
// the copy engine fills slot (L+1)%2 with layer L+1's experts.  Ordering
// uses only stream waits on events; the host never blocks.
#include <vector>

#include "internal.h"

namespace mxmoe {

LayerWs layer_ws_layout(int T, int H, int I, int E, int k, int inter_dtype) {
  LayerWs w{};
  const size_t rows = (size_t)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  w.ids = take(rows * 4);
  w.w = take(rows * 4);
  w.off = take(((size_t)E + 1) * 4);
  w.perm_src = take(rows * 4);
  w.dest_row = take(rows * 4);
  const bool mx8 = inter_dtype == MOE_OUT_MXFP8_E4M3;
  w.inter = take(rows * (size_t)I * (mx8 ? 1 : 2));
  w.inter_scales = take(mx8 ? rows * (size_t)(I / 32) : 0);
  w.y = take(rows * (size_t)H * 2);
  w.permute_ws = take(permute_ws_bytes(T, E, k));
  w.gemm_ws = take(gemm_ws_bytes((int)rows, E));
  w.total = o;
  return w;
}

namespace {

moe_status validate_layer_sizes(int T, int H, int I, int E, int k, int layout, int act, int inter) {
  if (T < 0 || H < 1 || I < 1) return fail(MOE_ERR_SHAPE, "layer: T %d, H %d, I %d out of range", T, H, I);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "layer: E = %d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 64) return fail(MOE_ERR_SHAPE, "layer: k = %d outside [1, min(E, 64)]", k);
  if (H % 32 || I % 32)
    return fail(MOE_ERR_SHAPE, "layer: H (%d) and I (%d) must be multiples of the 32-element MX block", H, I);
  if (layout != MOE_EPI_SWIGLU_SPLIT && layout != MOE_EPI_SWIGLU_INTERLEAVED)
    return fail(MOE_ERR_INVALID_ARG, "layer: layout %d is not a SwiGLU layout", layout);
  if (act != MOE_ACT_BF16 && act != MOE_ACT_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "layer: bad act_dtype %d", act);
  if (inter != MOE_OUT_BF16 && inter != MOE_OUT_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "layer: inter_dtype %d must be MOE_OUT_BF16 or MOE_OUT_MXFP8_E4M3", inter);
  if (inter == MOE_OUT_MXFP8_E4M3 && H % 512)
    return fail(MOE_ERR_NOT_IMPLEMENTED, "layer: an MXFP8 intermediate needs H %% 512 == 0 (H = %d)", H);
  if ((int64_t)T * k >= (1ll << 31)) return fail(MOE_ERR_SHAPE, "layer: T*k overflows int32");
  return MOE_OK;
}

// tiled weights: FC1 (K = H, N = 2I) and FC2 (K = I, N = H) must both be tileable
moe_status validate_w_format(int w_format, int H, int I) {
  if (w_format != MOE_W_CANONICAL && w_format != MOE_W_TILED)
    return fail(MOE_ERR_INVALID_ARG, "layer: bad w_format %d", w_format);
  if (w_format == MOE_W_TILED && (H % 512 || I % 512))
    return fail(MOE_ERR_SHAPE, "layer: tiled weights need H %% 512 == 0 and I %% 512 == 0 (H %d, I %d)", H, I);
  return MOE_OK;
}

// A layer's routing arrays (route + permute outputs) and the permutation's
// scratch.
struct Routing {
  int32_t* ids;
  float* w;
  int32_t* off;
  int32_t* perm_src;
  int32_t* dest_row;
  void* permute_ws;
};

Routing layer_routing(const LayerWs& L, uint8_t* ws) {
  Routing r{};
  r.ids = reinterpret_cast<int32_t*>(ws + L.ids);
  r.w = reinterpret_cast<float*>(ws + L.w);
  r.off = reinterpret_cast<int32_t*>(ws + L.off);
  r.perm_src = reinterpret_cast<int32_t*>(ws + L.perm_src);
  r.dest_row = reinterpret_cast<int32_t*>(ws + L.dest_row);
  r.permute_ws = ws + L.permute_ws;
  return r;
}

// Routing arrays alone (the streamed pass's per-slot copies).
struct RouteWs {
  size_t ids, w, off, perm_src, dest_row, permute_ws, total;
};

RouteWs route_ws_layout(int T, int E, int k) {
  RouteWs w{};
  const size_t rows = (size_t)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  w.ids = take(rows * 4);
  w.w = take(rows * 4);
  w.off = take(((size_t)E + 1) * 4);
  w.perm_src = take(rows * 4);
  w.dest_row = take(rows * 4);
  w.permute_ws = take(permute_ws_bytes(T, E, k));
  w.total = o;
  return w;
}

Routing slot_routing(const RouteWs& L, uint8_t* ws) {
  Routing r{};
  r.ids = reinterpret_cast<int32_t*>(ws + L.ids);
  r.w = reinterpret_cast<float*>(ws + L.w);
  r.off = reinterpret_cast<int32_t*>(ws + L.off);
  r.perm_src = reinterpret_cast<int32_t*>(ws + L.perm_src);
  r.dest_row = reinterpret_cast<int32_t*>(ws + L.dest_row);
  r.permute_ws = ws + L.permute_ws;
  return r;
}

moe_status run_routing(const float* logits, int T, int E, int k, const Routing& r, hipStream_t s) {
  MXMOE_TRY(launch_route(logits, T, E, k, r.ids, r.w, s));
  return launch_permute(r.ids, T, E, k, r.off, r.perm_src, r.dest_row, r.permute_ws, s);
}

// FC1 + SwiGLU -> FC2 -> combine of a routed layer, all arguments valid, T > 0;
// intermediate, FC2 output and GEMM scratch in a.workspace.  `reserve`: CUs
// per XCD the GEMMs leave free.  The routing picks k distinct experts per
// token, so no expert has more than T rows: the GEMMs skip the row-tile
// classes that need more (at T <= 32 only the 32-row class runs).
moe_status run_experts(const moe_layer_args& a, const Routing& r, hipStream_t s, int reserve) {
  const LayerWs L = layer_ws_layout(a.T, a.H, a.I, a.E, a.k, a.inter_dtype);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const int rows = a.T * a.k;

  moe_gemm_args g1{};
  g1.a = a.x;
  g1.a_scales = a.x_scales;
  g1.a_dtype = a.act_dtype;
  g1.a_gather = r.perm_src;
  g1.a_gather_div = a.k;
  g1.a_rows = a.T;
  g1.rows = rows;
  g1.w_packed = a.w1_packed;
  g1.w_scales = a.w1_scales;
  g1.expert_offsets = r.off;
  g1.E = a.E;
  g1.N = 2 * a.I;
  g1.K = a.H;
  g1.epilogue = a.layout;
  g1.c = ws + L.inter;
  g1.c_scales = a.inter_dtype == MOE_OUT_MXFP8_E4M3 ? ws + L.inter_scales : nullptr;
  g1.c_dtype = a.inter_dtype;
  g1.w_format = a.w_format;
  MXMOE_TRY(launch_gemm(g1, ws + L.gemm_ws, s, reserve, a.T));

  moe_gemm_args g2{};
  g2.a = ws + L.inter;
  g2.a_scales = g1.c_scales;
  g2.a_dtype = a.inter_dtype == MOE_OUT_MXFP8_E4M3 ? MOE_ACT_MXFP8_E4M3 : MOE_ACT_BF16;
  g2.a_gather = nullptr;
  g2.a_gather_div = 1;
  g2.a_rows = rows;
  g2.rows = rows;
  g2.w_packed = a.w2_packed;
  g2.w_scales = a.w2_scales;
  g2.expert_offsets = r.off;
  g2.E = a.E;
  g2.N = a.H;
  g2.K = a.I;
  g2.epilogue = MOE_EPI_NONE;
  g2.c = ws + L.y;
  g2.c_dtype = MOE_OUT_BF16;
  g2.w_format = a.w_format;
  MXMOE_TRY(launch_gemm(g2, ws + L.gemm_ws, s, reserve, a.T));

  return launch_combine(ws + L.y, MOE_OUT_BF16, r.dest_row, r.w, a.T, a.k, a.H, a.out, a.x_next, s);
}

// The body of a layer, all arguments valid; pointers into `ws`.
moe_status run_layer(const moe_layer_args& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  const LayerWs L = layer_ws_layout(a.T, a.H, a.I, a.E, a.k, a.inter_dtype);
  const Routing r = layer_routing(L, static_cast<uint8_t*>(a.workspace));
  MXMOE_TRY(run_routing(a.logits, a.T, a.E, a.k, r, s));
  return run_experts(a, r, s, 0);
}

struct BlobLayout {
  size_t w1p, s1, w2p, s2, total;
};

BlobLayout blob_layout(int H, int I, int E) {
  BlobLayout b{};
  const size_t e = (size_t)E;
  size_t o = 0;
  b.w1p = o; o = align_up(o + e * 2 * I * (H / 2), 256);
  b.s1 = o;  o = align_up(o + e * 2 * I * (H / 32), 256);
  b.w2p = o; o = align_up(o + e * H * (I / 2), 256);
  b.s2 = o;  o = align_up(o + e * H * (I / 32), 256);
  b.total = o;
  return b;
}

// Streamed-pass workspace: one layer workspace, the fp32 output of inner
// layers, two bf16 chain buffers, and per slot the routing arrays of the
// routed expert copy (laid out as the routing part of a layer workspace).
struct StreamWs {
  size_t layer, out_tmp, xbuf0, xbuf1, route[2], route_bytes, total;
};

StreamWs stream_ws_layout(int T, int H, int I, int E, int k) {
  StreamWs s{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  s.layer = take(layer_ws_layout(T, H, I, E, k, MOE_OUT_BF16).total);
  s.out_tmp = take((size_t)T * H * 4);
  s.xbuf0 = take((size_t)T * H * 2);
  s.xbuf1 = take((size_t)T * H * 2);
  s.route_bytes = route_ws_layout(T, E, k).total;
  s.route[0] = take(s.route_bytes);
  s.route[1] = take(s.route_bytes);
  s.total = o;
  return s;
}

// Five events per (thread, device), created once and reused by every
// streamed call on that thread: a stream wait captures the event's state
// when it is enqueued, so re-recording in a later call is safe, and no
// event is ever destroyed while a stream may still wait on it.
moe_status stream_events(hipEvent_t** out) {
  static thread_local std::vector<std::vector<hipEvent_t>> pool;
  int dev = 0;
  MXMOE_HIP(hipGetDevice(&dev));
  if ((int)pool.size() <= dev) pool.resize(dev + 1);
  std::vector<hipEvent_t>& v = pool[dev];
  while (v.size() < 5) {
    hipEvent_t e;
    MXMOE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    v.push_back(e);
  }
  *out = v.data();
  return MOE_OK;
}

}  // namespace
}  // namespace mxmoe

using namespace mxmoe;

extern "C" {

size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t inter) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return 0;
  return layer_ws_layout(T, H, I, E, k, inter).total;
}

size_t moe_layer_workspace_offset(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t inter,
                                  int32_t which) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return (size_t)-1;
  const LayerWs L = layer_ws_layout(T, H, I, E, k, inter);
  switch (which) {
    case 0: return L.ids;
    case 1: return L.w;
    case 2: return L.off;
    case 3: return L.perm_src;
    case 4: return L.dest_row;
    default: return (size_t)-1;
  }
}

moe_status moe_layer_forward(const moe_layer_args* a, void* stream) {
  clear_error();
  if (!a) return fail(MOE_ERR_INVALID_ARG, "layer: null args");
  MXMOE_TRY(validate_layer_sizes(a->T, a->H, a->I, a->E, a->k, a->layout, a->act_dtype, a->inter_dtype));
  MXMOE_TRY(validate_w_format(a->w_format, a->H, a->I));
  if (a->T > 0 && (!a->logits || !a->x || !a->w1_packed || !a->w1_scales || !a->w2_packed ||
                   !a->w2_scales || !a->out))
    return fail(MOE_ERR_INVALID_ARG, "layer: null pointer");
  if (a->act_dtype == MOE_ACT_MXFP8_E4M3 && a->T > 0 && !a->x_scales)
    return fail(MOE_ERR_INVALID_ARG, "layer: MXFP8 x needs x_scales");
  const size_t need = layer_ws_layout(a->T, a->H, a->I, a->E, a->k, a->inter_dtype).total;
  if (!a->workspace || a->workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "layer: workspace %zu bytes, need %zu", a->workspace_bytes, need);
  MXMOE_TRY(check_device());
  return run_layer(*a, (hipStream_t)stream);
}

size_t moe_blob_bytes(int32_t H, int32_t I, int32_t E) {
  if (H < 1 || I < 1 || E < 1) return 0;
  return blob_layout(H, I, E).total;
}

size_t moe_blob_section_offset(int32_t H, int32_t I, int32_t E, int32_t which) {
  if (H < 1 || I < 1 || E < 1) return (size_t)-1;
  const BlobLayout b = blob_layout(H, I, E);
  switch (which) {
    case 0: return b.w1p;
    case 1: return b.s1;
    case 2: return b.w2p;
    case 3: return b.s2;
    default: return (size_t)-1;
  }
}

size_t moe_streamed_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return 0;
  return stream_ws_layout(T, H, I, E, k).total;
}

moe_status moe_layer_prefill_streamed(const moe_streamed_args* a, void* compute_stream, void* copy_stream) {
  clear_error();
  if (!a) return fail(MOE_ERR_INVALID_ARG, "streamed: null args");
  MXMOE_TRY(validate_layer_sizes(a->T, a->H, a->I, a->E, a->k, a->layout, MOE_ACT_BF16, MOE_OUT_BF16));
  MXMOE_TRY(validate_w_format(a->w_format, a->H, a->I));
  if (a->num_layers < 1) return fail(MOE_ERR_SHAPE, "streamed: num_layers = %d < 1", a->num_layers);
  if (a->depth != 1 && a->depth != 2) return fail(MOE_ERR_INVALID_ARG, "streamed: depth %d must be 1 or 2", a->depth);
  if (a->chain != MOE_CHAIN_RMS && a->chain != MOE_CHAIN_INDEPENDENT)
    return fail(MOE_ERR_INVALID_ARG, "streamed: bad chain %d", a->chain);
  if (a->expert_copy != MOE_COPY_ALL && a->expert_copy != MOE_COPY_ROUTED && a->expert_copy != MOE_COPY_AUTO)
    return fail(MOE_ERR_INVALID_ARG, "streamed: bad expert_copy %d", a->expert_copy);
  if (a->routed_copy_max_tokens < 0)
    return fail(MOE_ERR_INVALID_ARG, "streamed: routed_copy_max_tokens %d < 0", a->routed_copy_max_tokens);
  const bool routed = a->expert_copy == MOE_COPY_ROUTED ||
                      (a->expert_copy == MOE_COPY_AUTO && a->T <= a->routed_copy_max_tokens);
  if (a->num_blobs < 1 || !a->host_blobs) return fail(MOE_ERR_INVALID_ARG, "streamed: no host blobs");
  if (!a->device_slot[0] || (a->depth == 2 && !a->device_slot[1]))
    return fail(MOE_ERR_INVALID_ARG, "streamed: device slot missing");
  if (!a->logits || !a->x || !a->out) return fail(MOE_ERR_INVALID_ARG, "streamed: null pointer");
  const BlobLayout bl = blob_layout(a->H, a->I, a->E);
  if (a->blob_bytes < bl.total)
    return fail(MOE_ERR_SHAPE, "streamed: blob_bytes %zu < %zu needed", a->blob_bytes, bl.total);
  const StreamWs sw = stream_ws_layout(a->T, a->H, a->I, a->E, a->k);
  if (!a->workspace || a->workspace_bytes < sw.total)
    return fail(MOE_ERR_WORKSPACE, "streamed: workspace %zu bytes, need %zu", a->workspace_bytes, sw.total);
  for (int b = 0; b < a->num_blobs; ++b) {
    if (!a->host_blobs[b]) return fail(MOE_ERR_INVALID_ARG, "streamed: host blob %d is null", b);
    if (routed && reinterpret_cast<uintptr_t>(a->host_blobs[b]) % 16)
      return fail(MOE_ERR_INVALID_ARG, "streamed: routed copy needs 16-byte aligned blobs (blob %d)", b);
  }
  for (int i = 0; i < a->depth; ++i)
    if (routed && reinterpret_cast<uintptr_t>(a->device_slot[i]) % 16)
      return fail(MOE_ERR_INVALID_ARG, "streamed: routed copy needs 16-byte aligned slots (slot %d)", i);
  // one stream for both would run every copy after the previous layer's compute
  if (a->depth == 2 && compute_stream == copy_stream)
    return fail(MOE_ERR_INVALID_ARG,
                "streamed: depth 2 needs a copy stream distinct from the compute stream (one stream serialises "
                "the pipeline)");
  MXMOE_TRY(check_device());
  // the routed copy kernel reads each blob through the address the device
  // maps it at
  std::vector<const uint8_t*> dev_blob(a->num_blobs, nullptr);
  for (int b = 0; b < a->num_blobs; ++b) {
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, a->host_blobs[b]);
    (void)hipGetLastError();
    if (e != hipSuccess || attr.type != hipMemoryTypeHost)
      return fail(MOE_ERR_NOT_PINNED, "streamed: host blob %d is not page-locked host memory", b);
    if (routed) {
      if (!attr.devicePointer || attr.hostPointer != a->host_blobs[b])
        return fail(MOE_ERR_NOT_PINNED, "streamed: host blob %d has no device-mapped address", b);
      dev_blob[b] = static_cast<const uint8_t*>(attr.devicePointer);
    }
  }

  hipStream_t cs = (hipStream_t)compute_stream, xs = (hipStream_t)copy_stream;
  hipEvent_t* user_ev = static_cast<hipEvent_t*>(a->events);
  hipEvent_t* ev = nullptr;
  MXMOE_TRY(stream_events(&ev));
  hipEvent_t start = ev[0];
  hipEvent_t copied[2] = {ev[1], ev[2]};
  hipEvent_t computed[2] = {ev[3], ev[4]};

  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  const size_t TH = (size_t)a->T * a->H;
  const RouteWs rw = route_ws_layout(a->T, a->E, a->k);
  const Routing slot_route[2] = {slot_routing(rw, ws + sw.route[0]), slot_routing(rw, ws + sw.route[1])};
  // bytes of one expert in each blob section (contiguous per expert in both weight orders)
  const uint64_t per_expert[4] = {(uint64_t)2 * a->I * (a->H / 2), (uint64_t)2 * a->I * (a->H / 32),
                                  (uint64_t)a->H * (a->I / 2), (uint64_t)a->H * (a->I / 32)};
  const size_t sec[4] = {bl.w1p, bl.s1, bl.w2p, bl.s2};
  // GEMMs leave one CU per XCD to the copy kernel, which runs one block per XCD
  const int reserve = routed ? 1 : 0;
  constexpr int kCopyBlocks = 8;

  // the copy stream must not overwrite a slot an earlier call's compute still reads
  MXMOE_HIP(hipEventRecord(start, cs));
  MXMOE_HIP(hipStreamWaitEvent(xs, start, 0));

  const uint16_t* x_cur = a->x;
  for (int L = 0; L < a->num_layers; ++L) {
    const int slot = a->depth == 2 ? (L & 1) : 0;
    uint8_t* dst = static_cast<uint8_t*>(a->device_slot[slot]);
    const float* logits = a->logits + (size_t)L * a->T * a->E;
    // slot reuse: depth 2 waits for layer L-2, depth 1 for layer L-1
    const int prev = L - a->depth;
    if (prev >= 0) MXMOE_HIP(hipStreamWaitEvent(xs, computed[slot], 0));
    if (user_ev) MXMOE_HIP(hipEventRecord(user_ev[4 * L + 0], xs));
    if (routed) {
      // this layer's routing on the copy stream, then only its hit experts
      if (a->T > 0) {
        MXMOE_TRY(run_routing(logits, a->T, a->E, a->k, slot_route[slot], xs));
        const uint8_t* src[4];
        uint8_t* dsts[4];
        for (int i = 0; i < 4; ++i) {
          src[i] = dev_blob[L % a->num_blobs] + sec[i];
          dsts[i] = dst + sec[i];
        }
        MXMOE_TRY(launch_routed_copy(src, dsts, per_expert, slot_route[slot].off, a->E, kCopyBlocks, xs));
      }
    } else {
      MXMOE_HIP(hipMemcpyAsync(dst, a->host_blobs[L % a->num_blobs], bl.total, hipMemcpyHostToDevice, xs));
    }
    if (user_ev) MXMOE_HIP(hipEventRecord(user_ev[4 * L + 1], xs));
    MXMOE_HIP(hipEventRecord(copied[slot], xs));

    MXMOE_HIP(hipStreamWaitEvent(cs, copied[slot], 0));
    if (user_ev) MXMOE_HIP(hipEventRecord(user_ev[4 * L + 2], cs));
    const bool last = L + 1 == a->num_layers;
    uint16_t* x_next = nullptr;
    if (!last && a->chain == MOE_CHAIN_RMS)
      x_next = a->layer_inputs ? a->layer_inputs + (size_t)(L + 1) * TH
                               : reinterpret_cast<uint16_t*>(ws + ((L & 1) ? sw.xbuf0 : sw.xbuf1));
    if (a->layer_inputs && (L == 0 || a->chain == MOE_CHAIN_INDEPENDENT))
      MXMOE_HIP(hipMemcpyAsync(a->layer_inputs + (size_t)L * TH, a->x, TH * 2, hipMemcpyDeviceToDevice, cs));

    moe_layer_args la{};
    la.T = a->T; la.H = a->H; la.I = a->I; la.E = a->E; la.k = a->k;
    la.layout = a->layout;
    la.act_dtype = MOE_ACT_BF16;
    la.inter_dtype = MOE_OUT_BF16;
    la.logits = logits;
    la.x = x_cur;
    la.x_scales = nullptr;
    la.w1_packed = dst + bl.w1p;
    la.w1_scales = dst + bl.s1;
    la.w2_packed = dst + bl.w2p;
    la.w2_scales = dst + bl.s2;
    la.out = last ? a->out : reinterpret_cast<float*>(ws + sw.out_tmp);
    la.x_next = x_next;
    la.workspace = ws + sw.layer;
    la.workspace_bytes = sw.out_tmp - sw.layer;
    la.w_format = a->w_format;
    if (routed) {
      if (a->T > 0) MXMOE_TRY(run_experts(la, slot_route[slot], cs, reserve));
    } else {
      MXMOE_TRY(run_layer(la, cs));
    }
    if (user_ev) MXMOE_HIP(hipEventRecord(user_ev[4 * L + 3], cs));
    MXMOE_HIP(hipEventRecord(computed[slot], cs));
    if (a->chain == MOE_CHAIN_RMS && !last) x_cur = x_next;
  }
  return MOE_OK;
}

}  // extern "C"
