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

// One step of the wave maximum: max(v, v of the lane the DPP control names);
// lanes with no source compare against 0, below every key.
template <int CTRL>
__device__ inline uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Largest key of the wave, in every lane.  Row shifts by 1, 2, 4 and 8 leave
// each 16-lane row's maximum in its lane 15; the row-15 broadcast (to the next
// row) and the row-31 broadcast (to rows 2 and 3) carry the wave's maximum to
// lane 63, which readlane hands to every lane.  Register-to-register moves,
// no LDS round trip per step.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111>(v);   // row_shr:1
  v = dpp_max_step<0x112>(v);   // row_shr:2
  v = dpp_max_step<0x114>(v);   // row_shr:4
  v = dpp_max_step<0x118>(v);   // row_shr:8
  v = dpp_max_step<0x142>(v);   // row_bcast:15
  v = dpp_max_step<0x143>(v);   // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
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

  // all of a lane's logits in flight at once: an in-range (clamped) address
  // under a wave-uniform guard, keys formed only after every load is issued
  const int nv = (E + 63) / 64;
  float val[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) val[i] = i < nv ? row[min(i * 64 + lane, E - 1)] : 0.f;
  uint64_t cand[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = i * 64 + lane;
    cand[i] = (e < E) ? (((uint64_t)order_key(val[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e)) : 0ull;
  }

  int my_id = 0;
  uint32_t my_key = 0u;
  for (int j = 0; j < k; ++j) {
    // lane-local maximum as a tree (depth 4 instead of a chain of 16)
    uint64_t m[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) m[i] = cand[i];
#pragma unroll
    for (int w = kPerLane / 2; w > 0; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) m[i] = m[i + w] > m[i] ? m[i + w] : m[i];
    const uint64_t best = m[0];
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
