// Weighted top-k combine (the end of a fused MoE: "Kimi-K3 SM120 FlashInfer
// MXFP4 MoE", goal section):
//   out[t][h] = sum_{j ascending} w[t][j] * y[dest_row[t*k + j]][h]   (fp32)
// One workgroup per token; each thread owns 8 consecutive h (16-byte bf16
// or 32-byte fp32 loads), so every row of y is read once, coalesced, and
// no atomics are involved.  The workgroup is sized to the row (at most 1024
// threads for bf16 rows, 512 for fp32 ones, whose 32-byte loads take twice
// the registers; whole waves, every pass over the row full but the last), and a
// thread has up to 16 rows of y in flight.  Optionally also writes the next
// stacked layer's input bf16(out[t] / rms(out[t])).
#include "internal.h"

namespace mxmoe {
namespace {

// raw 8-element vectors: bf16 as one 16-byte load, fp32 as two
struct Raw8Bf16 { uint4 q; };
struct Raw8F32 { float4 a, b; };

__device__ inline Raw8Bf16 load_raw(const uint16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ inline Raw8F32 load_raw(const float* p) {
  return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}

__device__ inline void widen(const Raw8Bf16& r, float* v) {
  const uint32_t u[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ inline void widen(const Raw8F32& r, float* v) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}

__device__ inline void load8(const float* p, float* v) { widen(load_raw(p), v); }

__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if (f != f) return 0x7fc0u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Rows are fetched kBatch at a time before any is accumulated (more loads in
// flight per thread); the accumulation order stays j = 0, 1, ..., k-1.
constexpr int kBatch = 16;
template <typename YT>
constexpr int max_threads() { return sizeof(YT) == 2 ? 1024 : 512; }   // threads per token, at most
constexpr int kMaxWaves = 1024 / 64;

// Threads per token for rows of H elements: the fewest passes of at most
// max_threads threads over the H/8 vectors, then the fewest whole waves that
// cover a pass.
int combine_threads(int H, int max_threads) {
  const int nv = H / 8;
  const int passes = (nv + max_threads - 1) / max_threads;
  const int per_pass = (nv + passes - 1) / passes;
  return (per_pass + 63) / 64 * 64;
}

template <typename YT>
__global__ __launch_bounds__(max_threads<YT>()) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ w, int k, int H,
                                                      float* __restrict__ out,
                                                      uint16_t* __restrict__ x_next) {
  using Raw = decltype(load_raw(y));
  const int t = blockIdx.x;
  const int nv = H / 8;
  float* orow = out + (size_t)t * H;
  const int32_t* rows = dest_row + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  const int nthr = blockDim.x;
  float ss = 0.f;
  for (int v = threadIdx.x; v < nv; v += nthr) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      Raw raw[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (j0 + b < k) raw[b] = load_raw(y + (size_t)rows[j0 + b] * H + 8 * v);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (j0 + b < k) {
          const float wj = wt[j0 + b];
          float yv[8];
          widen(raw[b], yv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, yv[i], acc[i]);
        }
      }
    }
    *reinterpret_cast<float4*>(orow + 8 * v) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(orow + 8 * v + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(acc[i], acc[i], ss);
  }
  if (x_next == nullptr) return;  // uniform over the block
  __shared__ float red[kMaxWaves];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < nthr / 64; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)H);
  uint16_t* xrow = x_next + (size_t)t * H;
  for (int v = threadIdx.x; v < nv; v += nthr) {
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
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(T), dim3(combine_threads(H, max_threads<uint16_t>())), 0, s,
                       static_cast<const uint16_t*>(y), dest_row, w, k, H, out, x_next);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(combine_threads(H, max_threads<float>())), 0, s,
                       static_cast<const float*>(y), dest_row, w, k, H, out, x_next);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace mxmoe
