// Weighted top-k combine (the end of a fused MoE: "Kimi-K3 SM120 FlashInfer
// MXFP4 MoE", goal section):
//   out[t][h] = sum_{j ascending} w[t][j] * y[dest_row[t*k + j]][h]   (fp32)
// One workgroup per token; each thread owns 8 consecutive h (16-byte bf16
// or 32-byte fp32 loads), so every row of y is read once, coalesced, and
// no atomics are involved.  Optionally also writes the next stacked layer's
// input bf16(out[t] / rms(out[t])).
#include "internal.h"

namespace mxmoe {
namespace {

__device__ inline void load8(const uint16_t* p, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

__device__ inline void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if (f != f) return 0x7fc0u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

template <typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ w, int k, int H,
                                                      float* __restrict__ out,
                                                      uint16_t* __restrict__ x_next) {
  const int t = blockIdx.x;
  const int nv = H / 8;
  float* orow = out + (size_t)t * H;
  float ss = 0.f;
  for (int v = threadIdx.x; v < nv; v += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = dest_row[(size_t)t * k + j];
      const float wj = w[(size_t)t * k + j];
      float yv[8];
      load8(y + (size_t)r * H + 8 * v, yv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, yv[i], acc[i]);
    }
    *reinterpret_cast<float4*>(orow + 8 * v) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(orow + 8 * v + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(acc[i], acc[i], ss);
  }
  if (x_next == nullptr) return;  // uniform over the block
  __shared__ float red[4];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H);
  uint16_t* xrow = x_next + (size_t)t * H;
  for (int v = threadIdx.x; v < nv; v += 256) {
    float o[8];
    load8(orow + 8 * v, o);  // this thread's own writes
    uint4 q;
    q.x = bf16_rne(o[0] * inv) | (bf16_rne(o[1] * inv) << 16);
    q.y = bf16_rne(o[2] * inv) | (bf16_rne(o[3] * inv) << 16);
    q.z = bf16_rne(o[4] * inv) | (bf16_rne(o[5] * inv) << 16);
    q.w = bf16_rne(o[6] * inv) | (bf16_rne(o[7] * inv) << 16);
    *reinterpret_cast<uint4*>(xrow + 8 * v) = q;
  }
}

}  // namespace

moe_status launch_combine(const void* y, int y_dtype, const int32_t* dest_row, const float* w,
                          int T, int k, int H, float* out, uint16_t* x_next, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (y_dtype == MOE_OUT_BF16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(T), dim3(256), 0, s,
                       static_cast<const uint16_t*>(y), dest_row, w, k, H, out, x_next);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(256), 0, s,
                       static_cast<const float*>(y), dest_row, w, k, H, out, x_next);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace mxmoe
