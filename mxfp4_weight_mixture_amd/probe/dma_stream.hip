// Weight-stream probes: how fast blocks pull contiguous 16 KB chunks from HBM,
// the access pattern of the grouped GEMM's weight stream (a unit reads its
// n-tile's tiled weights one 16 KB stage after another).  Measurement
// tooling, not part of libmxmoe's ABI.
//
// Block u streams chunks c = 0 .. chunks-1 at byte ((u * chunks + c) * 16 KB)
// with four waves, one 1 KB instruction per wave per quarter of a chunk
// (16 bytes a lane), in one of two ways:
//   * into LDS with buffer_load ... lds (the GEMM's DMA), a ring of eight
//     16 KB buffers, at most `depth` chunks in flight (1..7);
//   * into registers with nontemporal 16-byte loads, `depth` chunks (1..4)
//     loaded before they are folded into one word per thread (written to
//     `out`, so that nothing is optimised away).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ __launch_bounds__(256) void dma_chunks_kernel(const uint8_t* __restrict__ buf, int chunks) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[8 * 16384];
  const int u = blockIdx.x;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0, (int)0xffffffff, 0x00020000);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  for (int c = 0; c < chunks; ++c) {
    const uint32_t base = (uint32_t)(((uint64_t)u * chunks + c) * 16384);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(ring + (c & 7) * 16384 + (j * 4 + wave) * 1024), 16,
          base + (j * 4 + wave) * 1024 + (tid & 63) * 16, 0, 0, 0);
    // at most DEPTH chunks (four instructions each) still in flight
    constexpr int N = 4 * (DEPTH - 1);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  }
  __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));
}

template <int DEPTH>
__global__ __launch_bounds__(256) void load_chunks_kernel(const v4u* __restrict__ buf, int chunks,
                                                          uint32_t* __restrict__ out) {
  const int u = blockIdx.x;
  uint32_t acc = 0;
  for (int c0 = 0; c0 < chunks; c0 += DEPTH) {
    v4u v[DEPTH][4];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const uint64_t base = ((uint64_t)u * chunks + c0 + d) * 1024;   // in 16-byte pieces
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + d < chunks) v[d][j] = __builtin_nontemporal_load(buf + base + j * 256 + threadIdx.x);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + d < chunks) acc ^= v[d][j][0] ^ v[d][j][3];
  }
  out[(size_t)u * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Streams blocks * chunks 16 KB chunks of device buffer `buf` (at least
// blocks * chunks * 16 KB bytes, below 4 GiB) with `blocks` blocks; mode 0:
// global -> LDS DMA with depth 1..7 chunks in flight, mode 1: loads into
// registers, depth 1..4 (`out`: device uint32[blocks * 256]).  Returns the
// kernel time in ms (hipEvents on `stream`, synchronised), or a negative
// value on a HIP error or a bad argument.
float mxmoe_probe_chunk_stream(const void* buf, uint64_t buf_bytes, int blocks, int chunks, int mode, int depth,
                               uint32_t* out, void* stream) {
  if (!buf || blocks < 1 || chunks < 1) return -2.f;
  const uint64_t need = (uint64_t)blocks * (uint64_t)chunks * 16384u;
  if (need > buf_bytes || need > 0xffffffffull) return -2.f;
  if (mode == 0 ? (depth < 1 || depth > 7 || depth == 5) : (mode != 1 || !out || depth < 1 || depth > 4)) return -2.f;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) return -1.f;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  const v4u* v = static_cast<const v4u*>(buf);
  (void)hipEventRecord(e0, s);
  if (mode == 0) {
    switch (depth) {
      case 1: hipLaunchKernelGGL(dma_chunks_kernel<1>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
      case 2: hipLaunchKernelGGL(dma_chunks_kernel<2>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
      case 3: hipLaunchKernelGGL(dma_chunks_kernel<3>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
      case 4: hipLaunchKernelGGL(dma_chunks_kernel<4>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
      case 6: hipLaunchKernelGGL(dma_chunks_kernel<6>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
      default: hipLaunchKernelGGL(dma_chunks_kernel<7>, dim3(blocks), dim3(256), 0, s, b, chunks); break;
    }
  } else {
    switch (depth) {
      case 1: hipLaunchKernelGGL(load_chunks_kernel<1>, dim3(blocks), dim3(256), 0, s, v, chunks, out); break;
      case 2: hipLaunchKernelGGL(load_chunks_kernel<2>, dim3(blocks), dim3(256), 0, s, v, chunks, out); break;
      case 3: hipLaunchKernelGGL(load_chunks_kernel<3>, dim3(blocks), dim3(256), 0, s, v, chunks, out); break;
      default: hipLaunchKernelGGL(load_chunks_kernel<4>, dim3(blocks), dim3(256), 0, s, v, chunks, out); break;
    }
  }
  (void)hipEventRecord(e1, s);
  float ms = -1.f;
  if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess)
    (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

}  // extern "C"
