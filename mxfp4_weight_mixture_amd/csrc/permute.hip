// Stable counting sort of the T*k (token, slot) pairs by expert: the
// dispatch of routed tokens to the expert compute (ktransformers issue
// #2172, "Impact").  Rows of one expert keep increasing flat index
// f = t*k + j, so the result is unique and bit-exact.
//
//   1. histogram: one workgroup per chunk of kChunk flat entries counts its
//      experts in an LDS histogram (LDS atomics: order-free counts);
//   2. scan: one workgroup turns the [chunk][expert] counts into each
//      chunk's first row per expert (expert-major exclusive prefix), and
//      writes expert_offsets;
//   3. scatter: one wavefront per chunk walks its entries 64 at a time in
//      order.  Lanes holding the same expert are grouped with a ballot;
//      each lane's rank is the popcount of same-expert lanes below it, so
//      ties keep flat-index order without any global atomics.
#include "internal.h"

namespace mxmoe {
namespace {

constexpr int kChunk = 1024;

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                   int32_t* __restrict__ counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int f = base + i;
    if (f < n) atomicAdd(&hist[ids[f]], 1);
  }
  __syncthreads();
  int32_t* out = counts + (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += 256) out[e] = hist[e];
}

// inclusive scan over a 1024-thread block
__device__ inline int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) wave_tot[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int t = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(t, off, 64);
      if (lane >= off) t += o;
    }
    if (lane < 16) wave_tot[lane] = t;
  }
  __syncthreads();
  const int r = v + (wid > 0 ? wave_tot[wid - 1] : 0);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ counts, int nchunks,
                                                    int E, int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int tot = 0;
    if (e < E)
      for (int c = 0; c < nchunks; ++c) tot += counts[(size_t)c * E + e];
    const int incl = block_inclusive_scan(tot, wave_tot);
    const int base = carry + incl - tot;
    if (e < E) {
      offsets[e] = base;
      int run = base;
      for (int c = 0; c < nchunks; ++c) {
        const size_t i = (size_t)c * E + e;
        const int v = counts[i];
        counts[i] = run;
        run += v;
      }
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry += incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                     const int32_t* __restrict__ chunk_first,
                                                     int32_t* __restrict__ perm_src,
                                                     int32_t* __restrict__ dest_row) {
  extern __shared__ int pos[];
  const int lane = threadIdx.x;
  const int32_t* first = chunk_first + (size_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) pos[e] = first[e];
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int s = 0; s < kChunk; s += 64) {
    const int f = base + s + lane;
    const bool valid = f < n;
    const int e = valid ? ids[f] : -1;
    uint64_t pending = __ballot(valid);
    while (pending) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int le = __shfl(e, leader, 64);
      const uint64_t same = __ballot(e == le);
      const int p0 = pos[le];  // wave-uniform address
      if (e == le) {
        const int row = p0 + __popcll(same & ((1ull << lane) - 1ull));
        perm_src[row] = f;
        dest_row[f] = row;
      }
      if (lane == leader) pos[le] = p0 + __popcll(same);
      pending &= ~same;
    }
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t nchunks = (n + kChunk - 1) / kChunk;
  return align_up(nchunks * (size_t)E * sizeof(int32_t), 256) + 256;
}

moe_status launch_permute(const int32_t* ids, int T, int E, int k, int32_t* off,
                          int32_t* perm_src, int32_t* dest_row, void* ws, hipStream_t s) {
  const int n = T * k;
  const int nchunks = (n + kChunk - 1) / kChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)E * sizeof(int);
  if (nchunks > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), lds, s, ids, n, E, counts);
    MXMOE_HIP(hipGetLastError());
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, nchunks, E, off);
  MXMOE_HIP(hipGetLastError());
  if (nchunks > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(64), lds, s, ids, n, E, counts, perm_src,
                       dest_row);
    MXMOE_HIP(hipGetLastError());
  }
  return MOE_OK;
}

}  // namespace mxmoe
