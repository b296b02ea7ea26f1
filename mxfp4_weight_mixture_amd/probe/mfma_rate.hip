// Issue-rate probe of the gfx950 matrix instructions the grouped GEMM uses:
// the scaled 32x32x64 MFMA with FP8 (E4M3) x FP4 (E2M1) or FP4 x FP4
// operands, and the bf16 32x32x16 MFMA.  Measurement tooling, not part of
// libmxmoe's ABI: it sets the ceilings the GEMM's roofline is read against.
//
// Every wave runs `iters` rounds of eight products (eight independent
// accumulator chains) on register operands.  With `vary` set, both operands' bits change every round
// (an xor with a per-round constant, on the vector ALU beside the matrix
// core), as in a GEMM streaming random data; otherwise they stay constant.
// The accumulators are summed into `out` (one float per thread) so that
// nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two operand sets used alternately, eight accumulators: the xor that changes
// one set runs while the matrix core works on the other, so no product waits
// on a vector write to its own operands.
template <int AF, int BF>
__global__ __launch_bounds__(256) void scaled_kernel(int iters, int vary, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  v8i a0, b0, a1, b1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = (int)((t + 1) * 0x9E3779B9u + i * 0x85EBCA6Bu);
    b0[i] = (int)((t + 7) * 0xC2B2AE35u + i * 0x27D4EB2Fu);
    a1[i] = (int)((t + 3) * 0x27D4EB2Fu + i * 0x165667B1u);
    b1[i] = (int)((t + 5) * 0x85EBCA6Bu + i * 0x9E3779B9u);
  }
  // FP4 operands use the low four dwords only
  if (AF == 4) { a0[4] = a0[5] = a0[6] = a0[7] = 0; a1[4] = a1[5] = a1[6] = a1[7] = 0; }
  if (BF == 4) { b0[4] = b0[5] = b0[6] = b0[7] = 0; b1[4] = b1[5] = b1[6] = b1[7] = 0; }
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const int m = vary ? -1 : 0;
  for (int it = 0; it < iters; ++it) {
    const int k = (int)(0x9E3779B9u * (uint32_t)(it + 1)) & m;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc[j], AF, BF, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < (AF == 4 ? 4 : 8); ++i) a1[i] ^= k;
#pragma unroll
    for (int i = 0; i < (BF == 4 ? 4 : 8); ++i) b1[i] ^= k >> 1;
#pragma unroll
    for (int j = 4; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc[j], AF, BF, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < (AF == 4 ? 4 : 8); ++i) a0[i] ^= k >> 2;
#pragma unroll
    for (int i = 0; i < (BF == 4 ? 4 : 8); ++i) b0[i] ^= k >> 3;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[j][q];
  out[t] = s;
}

__global__ __launch_bounds__(256) void bf16_kernel(int iters, int vary, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  v4i a0, b0, a1, b1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // finite bf16 values
    a0[i] = (int)(((t + 1) * 0x9E3779B9u + i * 0x85EBCA6Bu) & 0x3fff3fffu);
    b0[i] = (int)(((t + 7) * 0xC2B2AE35u + i * 0x27D4EB2Fu) & 0x3fff3fffu);
    a1[i] = (int)(((t + 3) * 0x27D4EB2Fu + i * 0x165667B1u) & 0x3fff3fffu);
    b1[i] = (int)(((t + 5) * 0x85EBCA6Bu + i * 0x9E3779B9u) & 0x3fff3fffu);
  }
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const int m = vary ? 0x00ff00ff : 0;
  for (int it = 0; it < iters; ++it) {
    const int k = (int)(0x9E3779B9u * (uint32_t)(it + 1)) & m;
    v8bf xa, xb;
    __builtin_memcpy(&xa, &a0, 16);
    __builtin_memcpy(&xb, &b0, 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, xb, acc[j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a1[i] ^= k; b1[i] ^= k; }
    __builtin_memcpy(&xa, &a1, 16);
    __builtin_memcpy(&xb, &b1, 16);
#pragma unroll
    for (int j = 4; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, xb, acc[j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a0[i] ^= k; b0[i] ^= k; }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[j][q];
  out[t] = s;
}

}  // namespace

extern "C" {

// kind: 0 = FP8 x FP4 scaled, 1 = FP4 x FP4 scaled, 2 = bf16.  blocks of 256
// threads; `out` device float[blocks * 256].  Returns the kernel time in ms
// (hipEvents on `stream`, synchronised), or a negative value on a HIP error.
// Flops: 8 * iters * blocks * 4 waves * (2*32*32*64, or 2*32*32*16 for bf16).
float mxmoe_probe_mfma_rate(int kind, int blocks, int iters, int vary, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) return -1.f;
  hipEventRecord(e0, s);
  if (kind == 0) hipLaunchKernelGGL((scaled_kernel<0, 4>), dim3(blocks), dim3(256), 0, s, iters, vary, out);
  else if (kind == 1) hipLaunchKernelGGL((scaled_kernel<4, 4>), dim3(blocks), dim3(256), 0, s, iters, vary, out);
  else hipLaunchKernelGGL(bf16_kernel, dim3(blocks), dim3(256), 0, s, iters, vary, out);
  hipEventRecord(e1, s);
  float ms = -1.f;
  if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess) hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ms;
}

}  // extern "C"
