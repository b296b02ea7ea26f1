// HBM stream-read probe: the measured read bandwidth that the weight-streaming
// (small-token) shapes are read against beside the published 8 TB/s.
// Measurement tooling, not part of libmxmoe's ABI.
//
// Every thread walks the buffer in 16-byte pieces with a grid-wide stride
// (consecutive lanes take consecutive pieces, so a wave reads 1 KB per load
// instruction), UNROLL independent nontemporal loads in flight per thread,
// and folds what it read into one word (written to `out`, so that nothing
// is optimised away).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int UNROLL = 8;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ buf, uint64_t n16,
                                                          uint32_t* __restrict__ out) {
  const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t acc = 0;
  uint64_t i = tid;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    v4u v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[tid] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device buffer `buf` once with `blocks`
// blocks of 256 threads; `out` device uint32[blocks * 256].  Returns the
// kernel time in ms (hipEvents on `stream`, synchronised), or a negative
// value on a HIP error or a bad argument.
float mxmoe_probe_stream_read(const void* buf, uint64_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!buf || !out || blocks < 1 || bytes % 16) return -2.f;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) return -1.f;
  (void)hipEventRecord(e0, s);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const v4u*>(buf),
                     bytes / 16, out);
  (void)hipEventRecord(e1, s);
  float ms = -1.f;
  if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess)
    (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

}  // extern "C"
