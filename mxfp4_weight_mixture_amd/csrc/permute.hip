// Stable counting sort of the T*k (token, slot) pairs by expert: the
// dispatch of routed tokens to the expert compute (ktransformers issue
// #2172, "Impact").  Rows of one expert keep increasing flat index
// f = t*k + j, so the result is unique and bit-exact.
//
//   1. histogram: one workgroup per chunk of kChunk flat entries counts its
//      experts in an LDS histogram (LDS atomics: order-free counts);
//   2. column scan: one wavefront per expert turns that expert's counts
//      over the chunks into each chunk's first row relative to the expert
//      (exclusive prefix, 64 chunks per step) and the expert's total;
//   3. scatter: one wavefront per chunk first scans the experts' totals
//      (every chunk needs the expert offsets; chunk 0 also writes them),
//      then walks its entries 64 at a time in order.  Lanes holding the
//      same expert are found with one ballot per bit of the expert id (the
//      AND over the bits of "lanes whose bit agrees with mine"), so a step
//      costs the same however many distinct experts its 64 entries hold;
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

__device__ inline int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// counts[c][e] -> sum_{c' < c} counts[c'][e]; totals[e] = sum over all chunks
__global__ __launch_bounds__(256) void colscan_kernel(int32_t* __restrict__ counts, int nchunks, int E,
                                                      int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;  // whole wave
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nchunks ? counts[(size_t)c * E + e] : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (c < nchunks) counts[(size_t)c * E + e] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) totals[e] = carry;
}

// nchunks == 0 runs one block that only writes the (zero) offsets
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int n, int E, int nbits,
                                                     const int32_t* __restrict__ chunk_first,
                                                     const int32_t* __restrict__ totals,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm_src,
                                                     int32_t* __restrict__ dest_row) {
  extern __shared__ int pos[];
  const int lane = threadIdx.x;
  const bool has_entries = n > 0;
  const int32_t* first = chunk_first + (size_t)blockIdx.x * E;
  const int base = blockIdx.x * kChunk;
  // this chunk's ids, all in flight while the offsets are scanned below
  constexpr int kSteps = kChunk / 64;
  int idv[kSteps];
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int f = base + q * 64 + lane;
    idv[q] = f < n ? ids[f] : 0;
  }
  // the totals go through LDS first (independent loads, several in flight), so
  // that the scan below waits on LDS, not on a global load per 64 experts
#pragma unroll 8
  for (int e = lane; e < E; e += 64) pos[e] = totals[e];
  __syncthreads();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int v = e < E ? pos[e] : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (e < E) {
      const int start = carry + incl - v;
      pos[e] = start;
      if (blockIdx.x == 0) offsets[e] = start;
    }
    carry += __shfl(incl, 63, 64);
  }
  if (blockIdx.x == 0 && lane == 0) offsets[E] = carry;
  if (!has_entries) return;
  // this chunk's first row of each expert
#pragma unroll 8
  for (int e = lane; e < E; e += 64) pos[e] += first[e];
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int f = base + q * 64 + lane;
    const bool valid = f < n;
    const int e = idv[q];
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    // one LDS read per lane, then the lowest lane of each expert advances
    // that expert's position (a wave's LDS operations complete in order)
    const int p0 = valid ? pos[e] : 0;
    if (valid) {
      const int row = p0 + __popcll(same & below);
      perm_src[row] = f;
      dest_row[f] = row;
      if ((same & below) == 0) pos[e] = p0 + __popcll(same);
    }
  }
}

// All of a permutation that fits one chunk (n <= kChunk) in one block of 256
// threads: LDS histogram, block scan of the counts (each thread a run of
// consecutive experts), then the same stable scatter as scatter_kernel, by
// wave 0.  One launch instead of three for decode-sized batches.
__global__ __launch_bounds__(256) void permute_one_chunk_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                int nbits, int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm_src,
                                                                int32_t* __restrict__ dest_row) {
  extern __shared__ int pos[];
  __shared__ int wave_sum[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int e = tid; e < E; e += 256) pos[e] = 0;
  __syncthreads();
  for (int f = tid; f < n; f += 256) atomicAdd(&pos[ids[f]], 1);
  __syncthreads();
  // exclusive scan over the experts: thread tid owns experts [tid*R, tid*R + R)
  const int R = (E + 255) / 256;
  const int e0 = tid * R, e1 = min(E, e0 + R);
  int run = 0;
  for (int e = e0; e < e1; ++e) run += pos[e];
  const int incl = wave_inclusive_scan(run, lane);
  if (lane == 63) wave_sum[wid] = incl;
  __syncthreads();
  int start = incl - run;
  for (int w = 0; w < wid; ++w) start += wave_sum[w];
  for (int e = e0; e < e1; ++e) {
    const int c = pos[e];
    pos[e] = start;
    offsets[e] = start;
    start += c;
  }
  if (tid == 0) offsets[E] = n;
  __syncthreads();
  if (wid != 0) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int f = s0 + lane;
    const bool valid = f < n;
    const int e = valid ? ids[f] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int p0 = valid ? pos[e] : 0;
    if (valid) {
      const int row = p0 + __popcll(same & below);
      perm_src[row] = f;
      dest_row[f] = row;
      if ((same & below) == 0) pos[e] = p0 + __popcll(same);
    }
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t nchunks = (n + kChunk - 1) / kChunk;
  return align_up(nchunks * (size_t)E * sizeof(int32_t), 256) + align_up((size_t)E * sizeof(int32_t), 256);
}

moe_status launch_permute(const int32_t* ids, int T, int E, int k, int32_t* off,
                          int32_t* perm_src, int32_t* dest_row, void* ws, hipStream_t s) {
  const int n = T * k;
  const int nchunks = (n + kChunk - 1) / kChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* totals = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                               align_up((size_t)nchunks * E * sizeof(int32_t), 256));
  const size_t lds = (size_t)E * sizeof(int);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nchunks == 1) {
    hipLaunchKernelGGL(permute_one_chunk_kernel, dim3(1), dim3(256), lds, s, ids, n, E, nbits, off, perm_src,
                       dest_row);
    MXMOE_HIP(hipGetLastError());
    return MOE_OK;
  }
  if (nchunks > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), lds, s, ids, n, E, counts);
    MXMOE_HIP(hipGetLastError());
  }
  hipLaunchKernelGGL(colscan_kernel, dim3((E + 3) / 4), dim3(256), 0, s, counts, nchunks, E, totals);
  MXMOE_HIP(hipGetLastError());
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks > 0 ? nchunks : 1), dim3(64), lds, s, ids, n, E, nbits, counts,
                     totals, off, perm_src, dest_row);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace mxmoe
