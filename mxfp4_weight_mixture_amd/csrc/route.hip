// Top-k routing: one 64-lane wavefront per token.
//
// The router of a top-k MoE (256 experts / top-6 for DeepSeek-V4-Flash:
// ktransformers issue #2172, "Environment"; 896 / top-16 for Kimi-K3:
// "Kimi-K3 SM120 FlashInfer MXFP4 MoE", Phase-0 audit table).  Softmax is
// monotone, so selection works on the fp32 logits directly; the weights are
// the softmax renormalised over the k kept experts.
//
// Each lane holds up to 16 logits (E <= 1024) as 64-bit sort keys
// (order-preserving integer image of the float, then the complement of the
// expert id), so one wave-wide max per round picks the largest logit with
// the lowest id on ties.  k rounds of: lane-local max over its registers,
// 6-step butterfly max over the wave, owner clears the winner.
#include "internal.h"

namespace mxmoe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kPerLane = kMaxE / 64;

// Monotone map float -> uint32 (larger float -> larger key).  -0 == +0;
// NaN maps to 0, below every number (including -inf, whose key is 0x007fffff).
__device__ inline uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (v != v) return 0u;
  if ((b & 0x7fffffffu) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of order_key: the logit back from its key (-0 comes back as +0 and a
// NaN as a NaN, which give the same weights).
__device__ inline float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;

  uint64_t cand[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = i * 64 + lane;
    cand[i] = (e < E) ? (((uint64_t)order_key(row[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e))
                      : 0ull;
  }

  int my_id = 0;
  uint32_t my_key = 0u;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) best = cand[i] > best ? cand[i] : best;
    const uint64_t win = wave_max_u64(best);
    // the id part is unique, so exactly one register of one lane holds `win`
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (cand[i] == win) cand[i] = 0ull;
    const int e = (int)(0xffffffffu - (uint32_t)(win & 0xffffffffu));
    if (lane == j) {
      my_id = e;
      my_key = (uint32_t)(win >> 32);
    }
  }
  // the value from the key: no dependent global load per round
  const float my_val = key_value(my_key);
  // max over all E is the first pick (NaN sorts last)
  const float m = __shfl(my_val, 0, 64);
  // exp(l_j - max) with the difference formed exactly in double
  const double p = (lane < k) ? exp((double)my_val - (double)m) : 0.0;
  const double s = wave_sum_f64(p);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = (float)(p / s);
  }
}

}  // namespace

moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int blocks = (T + 3) / 4;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(256), 0, s, logits, T, E, k, ids, w);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace mxmoe
