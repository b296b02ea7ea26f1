// A resident layer captured once into a HIP graph and replayed with one
// launch.  The Phase-1 gates of the "Kimi-K3 SM120 FlashInfer MXFP4 MoE"
// page (item 5) ask for graph capture and replay at token counts 1/2/8/32:
// at those sizes the layer is a handful of short kernels, and issuing them
// one by one (plus the host-side argument checks of every call) is a
// visible share of the layer's time.
//
// The graph holds the five steps of moe_layer_forward with every pointer of
// the arguments it was captured with; a replay reads whatever those buffers
// hold at that time.  The steps zero their own counters with kernels (no
// memset nodes), so a replay needs nothing cleared beforehand.
#include <new>

#include "internal.h"

struct moe_layer_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int device;
};

extern "C" {

moe_status moe_layer_graph_create(const moe_layer_args* args, void* stream, moe_layer_graph** out) {
  using namespace mxmoe;
  clear_error();
  if (!out) return fail(MOE_ERR_INVALID_ARG, "layer graph: null output handle");
  *out = nullptr;
  if (!args) return fail(MOE_ERR_INVALID_ARG, "layer graph: null args");
  if (!stream) return fail(MOE_ERR_INVALID_ARG, "layer graph: capture needs a created stream, not the null stream");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  MXMOE_HIP(hipGetDevice(&dev));
  MXMOE_TRY(check_device());
  MXMOE_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed));
  const moe_status st = moe_layer_forward(args, stream);
  hipGraph_t g = nullptr;
  const hipError_t end = hipStreamEndCapture(s, &g);
  if (st != MOE_OK) {   // forward's own message stays
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (end != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    return fail(MOE_ERR_HIP, "layer graph: hipStreamEndCapture failed: %s", hipGetErrorString(end));
  }
  // an empty batch captures nothing: give the graph one empty node so that
  // instantiating and launching it are well defined
  size_t nodes = 0;
  if (hipGraphGetNodes(g, nullptr, &nodes) == hipSuccess && nodes == 0) {
    hipGraphNode_t empty = nullptr;
    const hipError_t e0 = hipGraphAddEmptyNode(&empty, g, nullptr, 0);
    if (e0 != hipSuccess) {
      (void)hipGraphDestroy(g);
      return fail(MOE_ERR_HIP, "layer graph: hipGraphAddEmptyNode failed: %s", hipGetErrorString(e0));
    }
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t inst = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  if (inst != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(MOE_ERR_HIP, "layer graph: hipGraphInstantiate failed: %s", hipGetErrorString(inst));
  }
  moe_layer_graph* h = new (std::nothrow) moe_layer_graph{g, exec, dev};
  if (!h) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(g);
    return fail(MOE_ERR_INVALID_ARG, "layer graph: out of host memory");
  }
  *out = h;
  return MOE_OK;
}

moe_status moe_layer_graph_launch(moe_layer_graph* graph, void* stream) {
  using namespace mxmoe;
  clear_error();
  if (!graph) return fail(MOE_ERR_INVALID_ARG, "layer graph: null handle");
  int dev = 0;
  MXMOE_HIP(hipGetDevice(&dev));
  if (dev != graph->device)
    return fail(MOE_ERR_INVALID_ARG, "layer graph: captured on device %d, current device is %d", graph->device, dev);
  MXMOE_HIP(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_graph_destroy(moe_layer_graph* graph) {
  using namespace mxmoe;
  clear_error();
  if (!graph) return MOE_OK;
  const hipError_t a = hipGraphExecDestroy(graph->exec);
  const hipError_t b = hipGraphDestroy(graph->graph);
  delete graph;
  if (a != hipSuccess) return fail(MOE_ERR_HIP, "layer graph: hipGraphExecDestroy failed: %s", hipGetErrorString(a));
  if (b != hipSuccess) return fail(MOE_ERR_HIP, "layer graph: hipGraphDestroy failed: %s", hipGetErrorString(b));
  return MOE_OK;
}

}  // extern "C"
