// Expert-grouped GEMM with MXFP4 weights (FC1 with a fused SwiGLU
// epilogue, FC2 plain) for gfx950.
//
// FC1 of a gated activation is twice as wide as FC2's inner size ("Kimi-K3
// SM120 FlashInfer MXFP4 MoE", on-machine evidence: the "256 vs. 128"
// inter-size check); the gate/up row arrangement is an explicit argument
// (same page, Phase-1 gates, item 2).  Two operand paths:
//   * bf16 activations: the MXFP4 weight tile is expanded to bf16 in
//     registers with v_cvt_scalef32_pk_bf16_fp4 (exact: every E2M1 value
//     times a power of two in the E8M0 range used is a bf16 number), then
//     v_mfma_f32_32x32x16_bf16 -- the same dequantise-to-16-bit idea the
//     Ampere kernel uses (issue #2172, comment on the Marlin MoE template),
//     on CDNA4 matrix cores;
//   * MXFP8 activations: v_mfma_scale_f32_32x32x64_f8f6f4 with A = FP8 E4M3,
//     B = FP4 E2M1, and both E8M0 block scales applied inside the MFMA
//     (the MXFP8 x MXFP4 product of the Kimi-K3 page, goal section).
//
// Work decomposition.  A small planning kernel splits each expert's rows
// into full tiles (256 rows; 128 with bf16 activations) plus one remainder
// tile, and files every tile under one of four row-tile sizes (32, 64, 128,
// 256) so that an expert with a handful of rows (the decode shapes, the tail
// of a skewed routing) does not pay for 256 rows of matrix-core work.  A
// (tile, n-tile) unit is one 256-column slice of one row tile.  Units are
// dealt to the 8 XCDs in contiguous ranges (in groups of row tiles x all
// n-tiles, row tile fastest), so that the blocks sharing an XCD's L2 share A
// rows and weight tiles; inside a range blocks draw units with an atomic,
// and a block whose XCD is done takes the other XCDs' remaining units.  With
// MXFP8 activations and a 256-row class, one persistent launch runs every
// class (gemm_mixed_kernel: the <= 32-row units' weight stream under the
// full tiles' matrix-core work); otherwise one persistent launch per class
// (gemm_dma_kernel).
//
// K loop (K % 512 == 0): per 128-element K stage the A rows (gathered
// through the permutation), the weight rows and, every four stages, both
// scales' 16-byte groups go global -> LDS with buffer_load ... lds into a
// ring of three stage buffers, two stages ahead of the products, the LDS
// layout swizzled so that fragment reads are conflict-free.  Other K use the
// register-staged gemm_kernel (global -> registers -> padded LDS).
//
// MFMA operand layout used (32x32 tiles, measured on gfx950 with one-hot
// operands): lane l supplies row/column (l % 32).  For the scaled
// 32x32x64 MFMA, an FP4 B lane in half g = l/32 holds K [32g, 32g+32) (one
// whole MX block), an FP8 A lane in half g holds K [16g, 16g+16) followed by
// K [32+16g, 32+16g+16), and the E8M0 scale supplied by a lane in half g
// applies to K block g of its row/column.  For the bf16 32x32x16 MFMA a
// lane in half g holds K [8g, 8g+8).  Accumulator j of lane l is
// C[8*(j/4) + 4*(l/32) + j%4][l % 32].  The two operands share that lane
// layout, so the DMA kernels, which pass the weights as the first operand and
// the activations as the second, accumulate the transposed tile: lane l owns
// one output row, which makes the per-row MX block amax of the MXFP8 epilogue
// one exchange with the partner lane l ^ 32.
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace mxmoe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kBN = 256;          // columns of W per unit
constexpr int kThreads = 256;
constexpr int kAStride = 144;     // bytes per LDS A row (128 + 16 pad)
constexpr int kClasses = 4;       // row-tile sizes 32, 64, 128, 256
constexpr int kXcds = 8;

// Phase timers: measurement tooling, compiled in only with
// MXMOE_PHASE_TIMERS=1 (libmxmoe_phases.so; the library proper has none).
// Wave 0 of each unit loop reads the 100 MHz s_memrealtime clock at the
// boundaries of a unit's phases and adds the durations, per block and
// row-tile class, into g_phase: [0] the K loop (from the issue of its first
// stages to its last product), between two units [1] the barrier and the
// next unit's draw, [2] the epilogue up to the last staging write, [3] the
// next unit's set-up, its first DMA and a barrier, [4] the staging's
// read-back and stores, [5] a barrier, [6] the rest (the next unit's other
// stages; a direct epilogue's whole time); [7] units, [8] the first unit's
// set-up, [9] unit loops run, [10] the complement of the earliest loop
// start, [11] the latest loop end (raw clock values: max over the block).
#ifndef MXMOE_PHASE_TIMERS
#define MXMOE_PHASE_TIMERS 0
#endif
constexpr int kPhaseSlots = 12;
#if MXMOE_PHASE_TIMERS
constexpr int kPhaseBlocks = 2048;
__device__ unsigned long long g_phase[kPhaseBlocks][kClasses][kPhaseSlots];
#endif

struct PhaseClock {
#if MXMOE_PHASE_TIMERS
  unsigned long long entry, last, d[7] = {0, 0, 0, 0, 0, 0, 0}, units = 0, setup = 0;
  __device__ PhaseClock() { entry = last = __builtin_amdgcn_s_memrealtime(); }
  // the first unit's stages are issued: its K loop starts
  __device__ void loop_start() {
    last = __builtin_amdgcn_s_memrealtime();
    setup = last - entry;
  }
  // phase i ends now
  __device__ void lap(int i) {
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    d[i] += t - last;
    last = t;
    if (i == 0) ++units;
  }
  __device__ void flush(int cls, bool record) {
    if (!record || blockIdx.x >= kPhaseBlocks) return;
    unsigned long long* g = g_phase[blockIdx.x][cls];
    for (int i = 0; i < 7; ++i) atomicAdd(g + i, d[i]);
    atomicAdd(g + 7, units);
    atomicAdd(g + 8, setup);
    atomicAdd(g + 9, 1ull);
    atomicMax(g + 10, ~entry);
    atomicMax(g + 11, (unsigned long long)__builtin_amdgcn_s_memrealtime());
  }
#else
  __device__ void loop_start() {}
  __device__ void lap(int) {}
  __device__ void flush(int, bool) {}
#endif
};

struct Tile {
  int expert;
  int row0;
};

struct Params {
  const uint8_t* a;
  const uint8_t* a_scales;
  const int32_t* a_gather;
  const uint8_t* w;
  const uint8_t* w_scales;
  const int32_t* offsets;
  void* c;
  uint8_t* c_scales;   // E8M0 [rows][n_out / 32], MXFP8 output only
  const Tile* tiles;
  const int32_t* tile_count;
  int32_t* unit_ctr;          // [8] per-XCD unit counters of this launch (zeroed by the planner)
  int tile_cap;               // the mixed launch: stride between the classes' tile lists
  int a_gather_div;
  uint32_t a_bytes, as_bytes;  // gathered A: bytes of A and of its scales from their starts (< 2^32)
  int N, K, n_out, n_tiles;
  int layout;  // 0 none, 1 split, 2 interleaved
};

__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if (f != f) return 0x7fc0u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// E8M0 byte -> fp32 2^(b-127); 0 -> 2^-127 (subnormal), 255 -> NaN
__device__ inline float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b == 0u ? 0x00400000u : (b == 255u ? 0x7fc00000u : (b << 23)));
}

template <int BM, bool FP8>
struct Cfg {
  static constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = kBN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int FN = WN / 32;
  static constexpr int KS = FP8 ? 128 : 64;         // K elements per stage
  static constexpr int BROW = KS / 2;               // packed B bytes per row per stage
  static constexpr int BSTRIDE = BROW + 16;
  static constexpr int SBLK = KS / 32;              // scale blocks per stage
  static constexpr int A_CHUNKS = BM * 8 / kThreads;        // 16-byte A chunks per thread
  static constexpr int B_CPR = BROW / 16;                   // 16-byte B chunks per row
  static constexpr int B_CHUNKS = kBN * B_CPR / kThreads;   // per thread
  static constexpr int LDS_A = BM * kAStride;
  static constexpr int LDS_B = kBN * BSTRIDE;
  static constexpr int LDS_AS = FP8 ? BM * 4 : 0;
  static constexpr int LDS_BS = kBN * 4;
  static constexpr int LDS_BUF = LDS_A + LDS_B + LDS_AS + LDS_BS;
};

// Row of W (within one expert) that feeds tile column j of n-tile nt.  The
// DMA kernels (and the tiled weight order) use groups of kSwiGroup = 64
// columns for every tile class; the register-staged kernels use their
// wave width.
constexpr int kSwiGroup = 64;
template <int WN>
__device__ inline int w_row_of(int layout, int nt, int j, int N, int n_out) {
  if (layout == 0) return min(nt * kBN + j, N - 1);
  // SwiGLU: each wave's WN columns are WN/2 gate rows then the WN/2 matching up
  // rows (selects only: the lane-dependent part has no branches)
  const int hp = WN / 2;
  const int i = nt * (kBN / 2) + (j / WN) * hp + (j % WN) % hp;
  const int up = (j % WN) >= hp ? 1 : 0;
  const int r = layout == 1 ? i + up * n_out : 2 * i + up;
  return i < n_out ? r : 0;
}

template <int BM, bool FP8, int EPI, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Params p) {
  using C = Cfg<BM, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::LDS_BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / C::WAVES_N) * C::WM;
  const int wn0 = (wave % C::WAVES_N) * C::WN;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int count = *p.tile_count;
  const int units = count * p.n_tiles;
  // contiguous unit ranges per XCD (blocks are dealt round-robin to XCDs)
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int u_end = min(units, (xcd + 1) * per_xcd);

  const int K = p.K;
  const int a_row_bytes = FP8 ? K : 2 * K;
  const int kb = K / 32;           // scale blocks per row
  const int nstages = (K + C::KS - 1) / C::KS;

  for (int u = xcd * per_xcd + slot; u < u_end; u += slots) {
    const int ti = u / p.n_tiles;
    const int nt = u % p.n_tiles;
    const Tile tile = p.tiles[ti];
    const int e = tile.expert;
    const int row0 = tile.row0;
    const int mrows = min(BM, p.offsets[e + 1] - row0);

    // ---- per-thread global sources (fixed over K) ----
    const uint8_t* a_src[C::A_CHUNKS];
    const int a_col = tid & 7;  // 16-byte column of the 128-byte stage row
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int grow = row0 + min(r, mrows - 1);
      const int arow = p.a_gather ? p.a_gather[grow] / p.a_gather_div : grow;
      a_src[i] = p.a + (size_t)arow * a_row_bytes + a_col * 16;
    }
    const uint8_t* as_src = nullptr;
    if (FP8 && tid < BM) {
      const int grow = row0 + min(tid, mrows - 1);
      const int arow = p.a_gather ? p.a_gather[grow] / p.a_gather_div : grow;
      as_src = p.a_scales + (size_t)arow * kb;
    }
    const uint8_t* b_src[C::B_CHUNKS];
    const int b_col = tid % C::B_CPR;
    const size_t w_expert = (size_t)e * p.N;
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      const int j = tid / C::B_CPR + (kThreads / C::B_CPR) * i;
      const int wr = w_row_of<C::WN>(p.layout, nt, j, p.N, p.n_out);
      b_src[i] = p.w + (w_expert + wr) * (size_t)(K / 2) + b_col * 16;
    }
    const uint8_t* bs_src;
    {
      const int wr = w_row_of<C::WN>(p.layout, nt, tid, p.N, p.n_out);
      bs_src = p.w_scales + (w_expert + wr) * (size_t)kb;
    }

    uint4 ra[C::A_CHUNKS];
    uint4 rb[C::B_CHUNKS];
    uint32_t ras = 0, rbs = 0;

    auto load_stage = [&](int s) {
      const int ka = s * 128;                 // A byte offset within the row
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i)
        ra[i] = (ka + a_col * 16 < a_row_bytes) ? *reinterpret_cast<const uint4*>(a_src[i] + ka)
                                                : make_uint4(0, 0, 0, 0);
      const int kbb = s * C::BROW;            // B byte offset within the row
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i)
        rb[i] = (kbb + b_col * 16 < K / 2) ? *reinterpret_cast<const uint4*>(b_src[i] + kbb)
                                           : make_uint4(0, 0, 0, 0);
      const int blk0 = s * C::SBLK;
      rbs = 0;
#pragma unroll
      for (int q = 0; q < C::SBLK; ++q)
        rbs |= (uint32_t)((blk0 + q < kb) ? bs_src[blk0 + q] : 127u) << (8 * q);
      if (FP8) {
        ras = 0;
        if (as_src) {
#pragma unroll
          for (int q = 0; q < C::SBLK; ++q)
            ras |= (uint32_t)((blk0 + q < kb) ? as_src[blk0 + q] : 127u) << (8 * q);
        }
      }
    };

    auto store_stage = [&](int buf) {
      uint8_t* base = lds + buf * C::LDS_BUF;
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *reinterpret_cast<uint4*>(base + r * kAStride + a_col * 16) = ra[i];
      }
      uint8_t* bb = base + C::LDS_A;
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) {
        const int j = tid / C::B_CPR + (kThreads / C::B_CPR) * i;
        *reinterpret_cast<uint4*>(bb + j * C::BSTRIDE + b_col * 16) = rb[i];
      }
      if (FP8 && tid < BM) *reinterpret_cast<uint32_t*>(base + C::LDS_A + C::LDS_B + tid * 4) = ras;
      *reinterpret_cast<uint32_t*>(base + C::LDS_A + C::LDS_B + C::LDS_AS + tid * 4) = rbs;
    };

    v16f acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int s = 0; s < nstages; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstages) load_stage(s + 1);
      const uint8_t* base = lds + buf * C::LDS_BUF;
      const uint8_t* la = base;
      const uint8_t* lb = base + C::LDS_A;
      const uint8_t* las = base + C::LDS_A + C::LDS_B;
      const uint8_t* lbs = las + C::LDS_AS;
      if constexpr (FP8) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          v8i af[C::FM];
          int asc[C::FM];
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm) {
            const int r = wm0 + fm * 32 + l32;
            // FP8 operand: lane half g carries K [16g, 16g+16) and [32+16g, 32+16g+16)
            // of this 64-wide step (half of each MX block), in that order.
            const uint8_t* src = la + r * kAStride + kk * 64 + g * 16;
            const v4i lo = *reinterpret_cast<const v4i*>(src);
            const v4i hi = *reinterpret_cast<const v4i*>(src + 32);
            af[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            asc[fm] = las[r * 4 + kk * 2 + g];
          }
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) {
            const int n = wn0 + fn * 32 + l32;
            const v4i bq = *reinterpret_cast<const v4i*>(lb + n * C::BSTRIDE + kk * 32 + g * 16);
            const v8i bf = v8i{bq[0], bq[1], bq[2], bq[3], 0, 0, 0, 0};
            const int bsc = lbs[n * 4 + kk * 2 + g];
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af[fm], bf, acc[fm][fn], 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, asc[fm], 0, bsc);
          }
        }
      } else {
        // expand this lane's 32 FP4 weights (one MX block) to bf16
        v8bf bw[C::FN][4];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int n = wn0 + fn * 32 + l32;
          const v4i bq = *reinterpret_cast<const v4i*>(lb + n * C::BSTRIDE + g * 16);
          const float sc = e8m0_to_f32(lbs[n * 4 + g]);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[d], sc, 0);
            const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[d], sc, 1);
            const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[d], sc, 2);
            const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[d], sc, 3);
            bw[fn][d] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          }
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          v8bf af[C::FM];
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm) {
            const int r = wm0 + fm * 32 + l32;
            af[fm] = *reinterpret_cast<const v8bf*>(la + r * kAStride + g * 64 + s4 * 16);
          }
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bw[fn][s4], acc[fm][fn],
                                                                    0, 0, 0);
        }
      }
      if (s + 1 < nstages) store_stage(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: registers -> C in permuted row order ----
    if constexpr (EPI == 0) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int n = nt * kBN + wn0 + fn * 32 + l32;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = wm0 + fm * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
            if (r < mrows && n < p.N) {
              const size_t o = (size_t)(row0 + r) * p.N + n;
              if (OUT == MOE_OUT_FP32) static_cast<float*>(p.c)[o] = acc[fm][fn][q];
              else static_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(acc[fm][fn][q]);
            }
          }
        }
    } else {
      constexpr int HF = C::FN / 2;
      const int i_base = nt * (kBN / 2) + (wave % C::WAVES_N) * (C::WN / 2);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fh = 0; fh < HF; ++fh) {
          const int i = i_base + fh * 32 + l32;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = wm0 + fm * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
            const float gv = acc[fm][fh][q];
            const float uv = acc[fm][fh + HF][q];
            const float a = gv / (1.0f + __expf(-gv)) * uv;
            if (r < mrows && i < p.n_out) {
              const size_t o = (size_t)(row0 + r) * p.n_out + i;
              if (OUT == MOE_OUT_FP32) static_cast<float*>(p.c)[o] = a;
              else static_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(a);
            }
          }
        }
    }
  }
}

// ---- main kernel: three-stage direct-to-LDS pipeline (K % 512 == 0) ----
//
// A stage covers 128 K elements: 4 MX blocks.  Every byte of a stage goes
// straight from global memory into LDS with global_load_lds_dwordx4, so
// three stages are in flight without staging registers: at iteration s the
// wave waits until its stage-s loads have landed (stage s+1's may still be
// in flight), one barrier publishes them and frees the buffer of stage s-1,
// the loads of stage s+2 are issued into that buffer, then stage s is
// multiplied.  E8M0 scales travel 16 bytes per row (four stages) at a time
// into a double-buffered scale area: a 4-byte-per-lane load costs about as
// much memory-pipeline time as a 16-byte one.
//
// LDS layout of a stage: A rows of RA bytes (128 for FP8, 256 for bf16), B
// rows of 64 bytes (two per 128-byte line).  A DMA instruction writes 64
// lanes x 16 bytes contiguously, so the layout is chosen through each
// lane's global address: slot j of a 128-byte window holds chunk j XOR a
// function of the row (or line) index, chosen so that the 16-byte fragment
// reads of any 16 consecutive rows (one LDS cycle of a 16-lane group) hit
// 16 different 16-byte bank groups, and any 8 consecutive rows 8 different
// ones, with no padding.

// Waves per block.  The full FP8 tiles run eight (two per SIMD, each wave a
// 64x128 slice): measured faster than four 128x128 waves.  The bf16 tiles
// run four: their waves expand their FP4 weights to bf16 on the vector ALU
// (v_cvt_scalef32_pk_bf16_fp4, two weights an instruction), and that
// expansion, not the matrix core, bounds them; a 128-row tile therefore
// gives each wave all 128 rows (128x64 slices), so that every expanded
// weight feeds four 32-row products.
template <int BM, bool FP8, int EPI>
constexpr int dma_waves() { return (BM == 256 && FP8) ? 8 : 4; }

template <int BM, bool FP8, int NWAVES = 4>
struct Cfg2 {
  static constexpr int NW = NWAVES;
  static constexpr int NT = NW * 64;
  static constexpr int WAVES_M = NW == 8 ? (BM == 256 ? 4 : 2) : (BM >= 128 && FP8 ? 2 : 1);
  static constexpr int WAVES_N = NW / WAVES_M;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = kBN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int FN = WN / 32;
  static constexpr int KS = 128;                    // K elements per stage
  static constexpr int RA = FP8 ? 128 : 256;        // A bytes per row per stage
  static constexpr int SA = RA / 16;                // 16-byte slots per A row
  static constexpr int RB = 64;                     // B bytes per row per stage
  static constexpr int NST = 3;
  static constexpr int LDS_A = BM * RA;
  static constexpr int LDS_B = kBN * RB;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static constexpr int SG_A = FP8 ? BM * 16 : 0;    // scale group: 16 bytes (4 stages) per row
  static constexpr int SG_B = kBN * 16;
  static constexpr int LDS_SG = SG_A + SG_B;
  static constexpr int LDS_TOTAL = NST * LDS_STAGE + 2 * LDS_SG;
  static constexpr int A_I = BM * RA / (NW * 1024);  // A DMA instructions per wave per stage
  static constexpr int B_I = kBN * RB / (NW * 1024);  // B DMA instructions per wave per stage
  static constexpr int A_ROWS_PER_I = 1024 / RA;    // A rows one instruction fills
  static constexpr int LOADS = A_I + B_I;           // data DMA instructions per wave per stage
  static_assert(LDS_TOTAL <= 163840, "LDS budget");
};

// swizzle of the 16-byte slots (see above)
template <bool FP8>
__device__ __forceinline__ int a_swz(int r) {
  return FP8 ? (((r >> 1) & 7) ^ ((r & 1) << 2)) : (r & 15);
}
__device__ __forceinline__ int b_swz(int line) { return ((line >> 1) & 3) ^ ((line & 1) << 1); }

// Raw buffer resource over [base, base + bytes) (4 GiB by default).  The DMA
// below addresses with a 32-bit per-lane offset plus a uniform (scalar) stage
// offset, which keeps one VGPR per load stream and no 64-bit address
// arithmetic in the loop; the host bounds every offset below 2^32.  A load
// at an offset past `bytes` is out of the resource's range: it returns zeros
// without a memory request (the tiles' padding rows use that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes = 0xffffffffu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane, global -> LDS (lane i writes dst + 16 i)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// This lane's index in its wave, in a fresh register each call: an opaque
// value (the compiler cannot hoist what is derived from it) that, unlike a
// copy of the thread index, keeps no register live between its uses.
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// LDS byte address of a pointer into this block's LDS
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS reads for code that runs while DMA into other LDS buffers is in flight:
// the compiler orders a plain LDS read after every outstanding LDS DMA (it
// cannot tell the buffers apart); these reads are outside its view, so each
// waits for its own data before it returns.
__device__ __forceinline__ uint4 lds_read16(uint32_t addr) {
  uint4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkm0() {
  // s_waitcnt lgkmcnt(0), vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroup barrier that also publishes this wave's LDS writes: s_barrier by
// itself does not wait for outstanding LDS operations, so without the
// lgkmcnt(0) another wave could read a location this wave's ds_write has not
// reached yet (DMA writes are waited for separately, with vmcnt).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// silu(g) * u with the hardware reciprocal (about 1 ulp) in place of an IEEE division
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Four fp32 values (|x| <= 448, which the MXFP8 scale below guarantees) ->
// four E4M3 codes, little-endian in one word, round to nearest even with
// E4M3 subnormals: the packed scaled conversion with scale 1.0.
typedef short short2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t e4m3x4_rne(float a, float b, float c, float d) {
  const short2_t z = {0, 0};
  const short2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, 1.0f, false);
  const short2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, c, d, 1.0f, false);
  // each result holds its two codes in the low half-word (first value in byte 0)
  return (uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)hi.x << 16);
}

// E8M0 exponent X of one MXFP8 block: the smallest X with amax * 2^-X <= 448
// (448 = 0.875 * 2^9), clamped to the E8M0 range; amax = 0 gives -127.
__device__ inline int mxfp8_block_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  const float f = frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1)
  const int x = f <= 0.875f ? e - 9 : e - 8;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// Output staging of one unit.  The accumulators hold the transposed tile
// (see the epilogue); MXFP8 output stages its E4M3 codes (one byte an
// element, quantised in registers) and each row's E8M0 bytes, bf16 output
// its values, fp32 output goes straight to memory.  A tile whose staging
// would cover more than two stage buffers is staged in row passes of whole
// waves, so that at least one stage buffer stays free while the epilogue
// runs.  The staging sits in the last USED stage buffers (from byte offset
// BASE on); the next unit's first PF stages go to buffers 0 .. PF-1, where
// they belong.
template <int BM, bool FP8, int EPI, int OUT, int NW>
struct EpiCfg {
  using C = Cfg2<BM, FP8, NW>;
  static constexpr bool MX = OUT == MOE_OUT_MXFP8_E4M3;
  static constexpr bool STAGED = OUT != MOE_OUT_FP32;
  static constexpr int TC = EPI == 0 ? kBN : kBN / 2;         // output columns of a tile
  static constexpr int PITCH = MX ? TC + 16 : 2 * TC + 16;    // staged bytes per row (16-byte pad)
  static constexpr int ROW_BYTES = MX ? PITCH + TC / 32 : PITCH;
  static constexpr int PASSES = !STAGED ? 0
                                : BM * ROW_BYTES <= 2 * C::LDS_STAGE       ? 1
                                : BM / 2 * ROW_BYTES <= 2 * C::LDS_STAGE   ? 2
                                                                           : 4;
  static constexpr int PROWS = STAGED ? BM / PASSES : 0;       // rows of one pass
  static constexpr int SC_OFF = PROWS * PITCH;                 // MXFP8: the rows' E8M0 bytes
  static constexpr int USED = (PROWS * ROW_BYTES + C::LDS_STAGE - 1) / C::LDS_STAGE;   // buffers staging covers
  static constexpr int PF = C::NST - USED;
  // whether the next unit's set-up and first PF stages start during the
  // epilogue (the eight-wave plain-output tiles keep no registers to spare
  // for the next unit's DMA offsets there: they start it after the epilogue)
  static constexpr bool EARLY = !(EPI == 0 && NW == 8);
  static constexpr int BASE = PF * C::LDS_STAGE;
  static_assert(!STAGED || (PASSES <= C::WAVES_M && C::WAVES_M % PASSES == 0), "passes of whole waves' rows");
  static_assert(PF >= 1, "a stage buffer stays free during the epilogue");
  static_assert(BASE + PROWS * ROW_BYTES <= C::NST * C::LDS_STAGE, "the staging stays within the stage buffers");
};

// One persistent block walks (tile, n-tile) units of one row-tile class: unit
// u, then the units next() returns (the same value in every thread; < 0: no
// more).  Per unit, the K loop runs over 128-element stages through three LDS
// stage buffers filled by DMA two stages ahead.  FP8 operands: the stage's
// fragments are read into registers half a stage ahead of their products
// (second k-half during the first half's MFMAs, next stage's first k-half
// during the second half's), with one barrier in the middle of each stage
// that both publishes stage s+1 and frees stage s's buffer for the DMA of
// stage s+3.  bf16 operands: the stage's reads and products follow one
// barrier at its start.  Between two units the next unit's scale group 0 and
// its first PF stages are issued into the LDS the epilogue's staging leaves
// free, once the staging is written and before it is read back and stored, so
// that their latency passes under the stores; its other stages follow the
// epilogue.
// next() may issue the block's following draw; settle(), called after each
// epilogue, takes its result.  tid_in: the thread's index within the NW waves
// that run the units; lds:
// their LDS area (Cfg2<BM, FP8, NW>::LDS_TOTAL bytes); store: false runs the
// units without writing C (a block that runs two units side by side keeps
// both halves in step with one).  Every wave of the block executes the same
// barriers, next() included.
template <int BM, bool FP8, int EPI, int OUT, bool TILED, int NW, typename Next, typename Settle>
__device__ __forceinline__ void run_units(const Params& p, int u, int count, int tid_in, uint8_t* lds, bool store,
                                          Next&& next, Settle&& settle) {
  using C = Cfg2<BM, FP8, NW>;
  using EC = EpiCfg<BM, FP8, EPI, OUT, NW>;
  const int K = p.K;
  const int a_row_bytes = FP8 ? K : 2 * K;
  const int kb = K / 32;
  const int nst = K / C::KS;
  // 32-column block of the tile that B fragment j of a wave reads.  Tile
  // columns come in groups of 64 (32 gate rows, then their 32 up rows) for
  // every tile class; the wave's fragments are ordered even blocks first, so
  // that with a SwiGLU epilogue fragment fh (gate) and fh + FN/2 (up) pair
  // up.  Without one the epilogue stages the same pairs side by side: that
  // order is also what keeps the eight-wave FC2 tile free of spills (its
  // identity order spilled 24-33 VGPRs of DMA offsets and LDS addresses
  // inside the K loop).
  auto frag_block = [](int j) { return (j % (C::FN / 2)) * 2 + j / (C::FN / 2); };
  uint8_t* const sg = lds + C::NST * C::LDS_STAGE;   // two scale groups

  // ---- DMA state of the unit whose stages are in flight (set by setup) ----
  int row0 = 0, mrows = 0, nt = 0;
  uint32_t a_off[C::A_I], b_off[C::B_I], as_off = 0, bs_off = 0;
  __amdgpu_buffer_rsrc_t ra, rb, ras, rbs;
  // scale loads: with four waves every wave loads 64 rows of A scales (if
  // below BM) and 64 of B scales; with eight, waves 0-3 load A, 4-7 load B
  const int wave_u = __builtin_amdgcn_readfirstlane(tid_in >> 6);
  const bool a_sw = C::NW == 8 ? wave_u < 4 : true;
  const bool b_sw = C::NW == 8 ? wave_u >= 4 : true;
  const int sw = (C::NW == 8 && wave_u >= 4) ? wave_u - 4 : wave_u;

  // Lane-derived values are recomputed wherever they are used, from
  // lane_id() and the wave index (a scalar).  Hoisted out of the unit loop
  // they stay live across it and get spilled, and a spill reload waits for
  // every DMA in flight.
  auto setup = [&](int uu) {
    const int lane = lane_id();
    const int wave = wave_u;
    // Units in groups of up to GM row tiles x all n-tiles, row tile fastest, so
    // that concurrent blocks of one XCD share their A rows and their weight
    // tiles.  The 256-row class holds a hot expert's full tiles one after
    // another (they share weights): GM = 4.  The other classes hold at most
    // one tile per expert (a remainder, or the one tile of a small expert), so
    // only A is shared, between the n-tiles of one row tile: GM = 1 (measured:
    // prefill256 and decode GEMMs 2-4 % faster, the 256-row class 7 % slower).
    constexpr int GM = BM == 256 ? 4 : 1;
    const int grp = uu / (GM * p.n_tiles);
    const int first = grp * GM;
    const int gsize = min(GM, count - first);
    const int in = uu - grp * GM * p.n_tiles;
    const int ti = first + in % gsize;
    nt = in / gsize;
    const Tile tile = p.tiles[ti];
    const int e = tile.expert;
    row0 = tile.row0;
    mrows = min(BM, p.offsets[e + 1] - row0);
    const size_t w_expert = (size_t)e * p.N;

    // DMA sources: uniform bases, 32-bit per-lane byte offsets (stage 0).
    // Gathered A rows: offsets from the start of A; contiguous A rows: from the
    // tile's first row.  In tiles of up to 64 rows the rows past the tile's
    // last one (most of a decode tile's 32 rows) load from the end of the A
    // resource's range, which reads zeros and moves no data; larger tiles
    // repeat their last row (rarely padded, and their K loop has no register
    // to spare for the range).
    constexpr bool kPadZero = BM <= 64;
    const bool gather = p.a_gather != nullptr;
    const uint8_t* const a_base = gather ? p.a : p.a + (size_t)row0 * a_row_bytes;
    const uint32_t a_nrec = !kPadZero ? 0xffffffffu : gather ? p.a_bytes : (uint32_t)mrows * (uint32_t)a_row_bytes;
    {
      int arow[C::A_I];
#pragma unroll
      for (int i = 0; i < C::A_I; ++i)
        arow[i] = min((wave * C::A_I + i) * C::A_ROWS_PER_I + lane / C::SA, mrows - 1);
      if (gather) {
        // all index loads in flight together
#pragma unroll
        for (int i = 0; i < C::A_I; ++i) arow[i] = p.a_gather[row0 + arow[i]];
#pragma unroll
        for (int i = 0; i < C::A_I; ++i) arow[i] /= p.a_gather_div;
      }
#pragma unroll
      for (int i = 0; i < C::A_I; ++i) {
        const int r = (wave * C::A_I + i) * C::A_ROWS_PER_I + lane / C::SA;
        const int chunk = (lane % C::SA) ^ a_swz<FP8>(r);
        a_off[i] = (!kPadZero || r < mrows) ? (uint32_t)arow[i] * (uint32_t)a_row_bytes + chunk * 16 : a_nrec;
      }
    }
    // B: canonical weights are addressed row by row (tile column j of the
    // stage's LDS layout <- its weight row); tiled weights already hold the
    // stage's 16 KB in LDS order, so each instruction copies 1 KB of
    // consecutive bytes.
    const size_t tile_id = (size_t)e * p.n_tiles + nt;
    const uint8_t* const b_base = TILED ? p.w + tile_id * (size_t)nst * C::LDS_B : p.w + w_expert * (size_t)(K / 2);
#pragma unroll
    for (int i = 0; i < C::B_I; ++i) {
      const int line = (wave * C::B_I + i) * 8 + lane / 8;
      const int uu2 = (lane & 7) ^ b_swz(line);
      const int j = line * 2 + (uu2 >> 2);
      const int wr = w_row_of<kSwiGroup>(p.layout, nt, j, p.N, p.n_out);
      b_off[i] = TILED ? (uint32_t)((wave * C::B_I + i) * 1024 + lane * 16)
                       : (uint32_t)wr * (uint32_t)(K / 2) + (uu2 & 3) * 16;
    }
    const int srow = sw * 64 + lane;   // scale row this lane loads (A: if < BM)
    const uint8_t* const as_base = gather ? p.a_scales : p.a_scales + (size_t)row0 * kb;
    const uint32_t as_nrec = !kPadZero ? 0xffffffffu : gather ? p.as_bytes : (uint32_t)mrows * (uint32_t)kb;
    as_off = kPadZero ? as_nrec : 0u;
    if (FP8 && a_sw && srow < (kPadZero ? mrows : BM)) {
      const int r = min(srow, mrows - 1);
      as_off = (uint32_t)(gather ? p.a_gather[row0 + r] / p.a_gather_div : r) * (uint32_t)kb;
    }
    const uint8_t* const bs_base =
        TILED ? p.w_scales + tile_id * (size_t)(K / 512) * 4096 : p.w_scales + w_expert * (size_t)kb;
    bs_off = TILED ? (uint32_t)(sw * 1024 + lane * 16)
                   : (uint32_t)w_row_of<kSwiGroup>(p.layout, nt, srow, p.N, p.n_out) * (uint32_t)kb;
    ra = make_rsrc(a_base, a_nrec);
    rb = make_rsrc(b_base);
    ras = make_rsrc(as_base, as_nrec);
    rbs = make_rsrc(bs_base);
  };
  // b_step / bs_step: bytes from one stage (one scale group) to the next
  const int b_step = TILED ? C::LDS_B : C::RB;
  const int bs_step = TILED ? 4096 : 16;
  auto stage_at = [&](int s) { return lds + __builtin_amdgcn_readfirstlane((s % C::NST) * C::LDS_STAGE); };
  auto issue = [&](int s) {
    uint8_t* base = stage_at(s);
#pragma unroll
    for (int i = 0; i < C::A_I; ++i) dma16(ra, a_off[i], s * C::RA, base + (wave_u * C::A_I + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_I; ++i)
      dma16(rb, b_off[i], s * b_step, base + C::LDS_A + (wave_u * C::B_I + i) * 1024);
  };
  // DMA instruction j of stage s (j < A_I: A, then B), for interleaving with products
  auto issue_one = [&](int s, int j) {
    uint8_t* base = stage_at(s);
    if (j < C::A_I) dma16(ra, a_off[j], s * C::RA, base + (wave_u * C::A_I + j) * 1024);
    else dma16(rb, b_off[j - C::A_I], s * b_step, base + C::LDS_A + (wave_u * C::B_I + j - C::A_I) * 1024);
  };
  // scale group j (stages 4j..4j+3): 16 bytes of every A and B row
  auto issue_scales = [&](int j) {
    uint8_t* base = sg + (j & 1) * C::LDS_SG;
    // (a 32-row tile has 512 bytes of A scales per group: lanes 32-63 stay idle)
    if (FP8 && a_sw && sw * 64 < BM && (BM >= 64 || lane_id() < BM)) dma16(ras, as_off, 16 * j, base + sw * 1024);
    if (b_sw) dma16(rbs, bs_off, bs_step * j, base + C::SG_A + sw * 1024);
  };

  PhaseClock clock;
  setup(__builtin_amdgcn_readfirstlane(u));
  issue_scales(0);
  issue(0);
  issue(1);
  issue(2);
  clock.loop_start();
  for (;;) {
    const int lane = lane_id();
    const int wave = wave_u;
    const int wm0 = (wave / C::WAVES_N) * C::WM;
    const int wn0 = (wave % C::WAVES_N) * C::WN;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    // fragment rows / lines start at multiples of 16, so the swizzles depend on the lane only
    const int xa = a_swz<FP8>(l32 & 15);
    const int xb = b_swz((l32 >> 1) & 7);

    v16f acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    if constexpr (FP8) {
      uint32_t sa[C::FM], sb[C::FN], na[C::FM], nb[C::FN];
      v8i a0[C::FM], a1[C::FM];
      v4i b0[C::FN], b1[C::FN];
      // LDS base of stage s, made opaque to the compiler: otherwise every
      // fragment address becomes an induction variable of its own
      auto stage_lds = [&](int s) {
        return lds + __builtin_amdgcn_readfirstlane((s % C::NST) * C::LDS_STAGE);
      };
      // read j of one k-half: j < FN: B fragment j; then the A fragments' low and high halves
      // (A: K [kk*64 + 16g, +16) and [kk*64 + 32 + 16g, +16) = chunks 4kk+g and 4kk+2+g)
      auto read_frag = [&](int s, int kk, int j, v8i (&af)[C::FM], v4i (&bq)[C::FN]) {
        const uint8_t* la = stage_lds(s);
        if (j < C::FN) {
          const int n = wn0 + frag_block(j) * 32 + l32;
          const int uu = ((n & 1) * 4 + 2 * kk + g) ^ xb;
          bq[j] = *reinterpret_cast<const v4i*>(la + C::LDS_A + (n >> 1) * 128 + (uu << 4));
        } else {
          const int fm = (j - C::FN) >> 1, hi = (j - C::FN) & 1;
          const uint8_t* row = la + (wm0 + fm * 32 + l32) * C::RA;
          const v4i v = *reinterpret_cast<const v4i*>(row + (((4 * kk + 2 * hi + g) ^ xa) << 4));
          if (hi) {
            af[fm][4] = v[0]; af[fm][5] = v[1]; af[fm][6] = v[2]; af[fm][7] = v[3];
          } else {
            af[fm][0] = v[0]; af[fm][1] = v[1]; af[fm][2] = v[2]; af[fm][3] = v[3];
          }
        }
      };
      // scale word j of stage s: four E8M0 bytes (the stage's blocks) of an A row or B column
      auto read_scale = [&](int s, int j, uint32_t (&ta)[C::FM], uint32_t (&tb)[C::FN]) {
        const uint8_t* lsg = sg + __builtin_amdgcn_readfirstlane(((s >> 2) & 1) * C::LDS_SG + (s & 3) * 4);
        if (j < C::FM) ta[j] = *reinterpret_cast<const uint32_t*>(lsg + (wm0 + j * 32 + l32) * 16);
        else tb[j - C::FM] = *reinterpret_cast<const uint32_t*>(lsg + C::SG_A + (wn0 + frag_block(j - C::FM) * 32 + l32) * 16);
      };
      // product i of one k-half, B-fragment major.  ta/tb hold this lane's scale
      // bytes in the order the op_sel field reads them: byte kk = block 2kk + g.
      // The weights are the instruction's first operand and the activations its
      // second, so the accumulator holds the transposed tile (see the epilogue).
      auto mma = [&](int kk, int i, const v8i (&af)[C::FM], const v4i (&bq)[C::FN], const uint32_t (&ta)[C::FM],
                     const uint32_t (&tb)[C::FN]) {
        const int fn = i / C::FM, fm = i % C::FM;
        const v8i bf = v8i{bq[fn][0], bq[fn][1], bq[fn][2], bq[fn][3], 0, 0, 0, 0};
        if (kk == 0)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af[fm], acc[fm][fn], 4 /*fp4 e2m1*/,
                                                                        0 /*fp8 e4m3*/, 0, tb[fn], 0, ta[fm]);
        else
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af[fm], acc[fm][fn], 4, 0, 1, tb[fn],
                                                                        1, ta[fm]);
      };
      // a stage's four scale bytes (blocks 0..3) -> this lane's two, in op_sel order
      const uint32_t scale_sel = g ? 0x0c0c0301u : 0x0c0c0200u;
      auto order_scales = [&](uint32_t (&ta)[C::FM], uint32_t (&tb)[C::FN]) {
#pragma unroll
        for (int j = 0; j < C::FM; ++j) ta[j] = __builtin_amdgcn_perm(0u, ta[j], scale_sel);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) tb[j] = __builtin_amdgcn_perm(0u, tb[j], scale_sel);
      };
      constexpr int MF = C::FM * C::FN;
      constexpr int NR = 2 * C::FM + C::FN;   // fragment reads of one k-half
      constexpr int NS = C::FM + C::FN;       // scale reads of one stage
      // reads issued after each product: at least two (front-loaded), more for small tiles
      constexpr int R1 = (NR + MF - 1) / MF > 2 ? (NR + MF - 1) / MF : 2;
      constexpr int R2 = (NR + NS + MF - 1) / MF > 2 ? (NR + NS + MF - 1) / MF : 2;
      constexpr int D2 = (C::LOADS + MF - 1) / MF;   // refill DMA instructions per product
      // One stage.  ISSUE: refill the freed buffer with stage s+3 during the second
      // half (SCALES: and the next scale group); WAIT: vmcnt allowance at the
      // mid-stage barrier, -1 for the last stage (no barrier, no next-stage
      // reads).  All three are compile-time constants so that the loop body has
      // no branch the compiler could sink the first half's products past.  Every
      // group of one product and its reads / DMA is fenced with sched_barrier to
      // keep the interleave.
      auto step = [&](int s, auto ISSUE, auto SCALES, auto WAIT, uint32_t (&ta)[C::FM], uint32_t (&tb)[C::FN],
                      uint32_t (&tna)[C::FM], uint32_t (&tnb)[C::FN]) {
        constexpr bool kIssue = decltype(ISSUE)::value;
        constexpr bool kScales = decltype(SCALES)::value;
        constexpr int kWait = decltype(WAIT)::value;
        order_scales(ta, tb);
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          mma(0, i, a0, b0, ta, tb);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = R1 * i; r < R1 * i + R1; ++r)
            if (r < NR) read_frag(s, 1, r, a1, b1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the first half's products stay ahead of the barrier
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) asm volatile("" : "+a"(acc[fm][fn]));
        if constexpr (kWait >= 0) {
          // stage s fully read by this wave; stage s+1 landed for this wave's loads
          wait_lgkm0();
          wait_vm<kWait>();
          stage_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          mma(1, i, a1, b1, ta, tb);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kWait >= 0) {
#pragma unroll
            for (int r = R2 * i; r < R2 * i + R2; ++r) {
              if (r < NS) read_scale(s + 1, r, tna, tnb);
              else if (r < NS + NR) read_frag(s + 1, 0, r - NS, a0, b0);
            }
          }
          // the refill of the freed buffer (stage s+3), spread over the products
          if constexpr (kIssue) {
#pragma unroll
            for (int j = D2 * i; j < D2 * i + D2; ++j) {
              if (j < C::LOADS) issue_one(s + 3, j);
              if (kScales && j == C::LOADS - 1) issue_scales((s + 3) >> 2);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      using T = std::integral_constant<bool, true>;
      using F = std::integral_constant<bool, false>;
      using WL = std::integral_constant<int, C::LOADS>;   // stage s+2 may still be in flight
      wait_vm<2 * C::LOADS>();
      stage_barrier();
#pragma unroll
      for (int r = 0; r < NS; ++r) read_scale(0, r, sa, sb);
#pragma unroll
      for (int r = 0; r < NR; ++r) read_frag(0, 0, r, a0, b0);
      // the stage count is a multiple of four (K % 512 == 0): groups of four stages,
      // the last group with its tail conditions resolved at compile time
      int s = 0;
      for (; s + 4 < nst; s += 4) {
        step(s, T{}, F{}, WL{}, sa, sb, na, nb);
        step(s + 1, T{}, T{}, WL{}, na, nb, sa, sb);
        step(s + 2, T{}, F{}, WL{}, sa, sb, na, nb);
        step(s + 3, T{}, F{}, WL{}, na, nb, sa, sb);
      }
      step(s, T{}, F{}, WL{}, sa, sb, na, nb);
      step(s + 1, F{}, F{}, WL{}, na, nb, sa, sb);
      step(s + 2, F{}, F{}, std::integral_constant<int, 0>{}, sa, sb, na, nb);
      step(s + 3, F{}, F{}, std::integral_constant<int, -1>{}, na, nb, sa, sb);
    } else {
      // bf16 A: the same pipeline as the FP8 path, with k-halves of 64 elements
      // (block h of each lane half), the weights expanded to bf16 in registers
      // (one conversion unit = 8 weights of one column, 4 instructions) spread
      // over the products of the preceding 16-element step.  FMA: the 32-row
      // fragments the unit's rows reach; the others' products and A reads are
      // left out (their accumulators stay zero and their rows are not stored).
      auto bf16_kloop = [&](auto fma_c) {
        constexpr int FMA = decltype(fma_c)::value;
        uint32_t sb[C::FN], nb[C::FN];
        v4i bqc[C::FN], bqn[C::FN];            // raw FP4 B of the current / next k-half
        v8bf afc[4][FMA], afn[4][FMA];         // A of the current / next k-half, per 16-element step
        v8bf bw[C::FN][4];                     // B of the current k-half, expanded
        auto stage_lds = [&](int s) {
          return lds + __builtin_amdgcn_readfirstlane((s % C::NST) * C::LDS_STAGE);
        };
        // read j of k-half h: j < FN: raw B of column fragment j; then A (step, fm)
        auto read_frag = [&](int s, int h, int j, v4i (&bq)[C::FN], v8bf (&af)[4][FMA]) {
          const uint8_t* la = stage_lds(s);
          if (j < C::FN) {
            const int n = wn0 + frag_block(j) * 32 + l32;
            const int uu = ((n & 1) * 4 + 2 * h + g) ^ xb;
            bq[j] = *reinterpret_cast<const v4i*>(la + C::LDS_A + (n >> 1) * 128 + (uu << 4));
          } else {
            const int s4 = (j - C::FN) / FMA, fm = (j - C::FN) % FMA;
            const uint8_t* row = la + (wm0 + fm * 32 + l32) * C::RA;
            // bytes 128h + 64g + 16*s4 of the 256-byte stage row: slot 8h + 4g + s4
            af[s4][fm] = *reinterpret_cast<const v8bf*>(row + (((8 * h + 4 * g + s4) ^ xa) << 4));
          }
        };
        auto read_scale = [&](int s, int j, uint32_t (&tb)[C::FN]) {
          const uint8_t* lsb = sg + __builtin_amdgcn_readfirstlane(((s >> 2) & 1) * C::LDS_SG + (s & 3) * 4) + C::SG_A;
          tb[j] = *reinterpret_cast<const uint32_t*>(lsb + (wn0 + frag_block(j) * 32 + l32) * 16);
        };
        // conversion unit (fn, d): the 8 weights of bw[fn][d] (E2M1 x block scale -> bf16, exact)
        auto expand = [&](int h, int fn, int d, const v4i (&bq)[C::FN], const uint32_t (&tb)[C::FN]) {
          const float sc = e8m0_to_f32((tb[fn] >> (8 * (2 * h + g))) & 0xff);
          const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[fn][d], sc, 0);
          const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[fn][d], sc, 1);
          const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[fn][d], sc, 2);
          const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)bq[fn][d], sc, 3);
          bw[fn][d] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        };
        constexpr int MG = C::FN * FMA;        // products of one 16-element step
        constexpr int MF = 4 * MG;             // products of one k-half
        constexpr int NR = C::FN + 4 * FMA;    // reads of one k-half
        constexpr int NS = C::FN;              // scale reads of one stage
        constexpr int R1 = (NR + MF - 1) / MF > 1 ? (NR + MF - 1) / MF : 1;
        constexpr int R2 = (NR + NS + MF - 1) / MF > 1 ? (NR + NS + MF - 1) / MF : 1;
        constexpr int D2 = (C::LOADS + MF - 1) / MF;
        // the products of k-half h from af/bq, with the expansion of step t+1's
        // weights after the MFMAs of step t (unit fn after the step's product fn*FM),
        // and EXTRA(i) (reads / DMA) after product i
        auto half = [&](int h, const v4i (&bq)[C::FN], const v8bf (&af)[4][FMA], const uint32_t (&tb)[C::FN],
                        auto&& extra) {
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) expand(h, fn, 0, bq, tb);
#pragma unroll
          for (int i = 0; i < MF; ++i) {
            const int s4 = i / MG, fn = (i % MG) / FMA, fm = i % FMA;
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[fn][s4], af[s4][fm], acc[fm][fn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (s4 < 3 && fm == 0) expand(h, fn, s4 + 1, bq, tb);
            extra(i);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        auto step = [&](int s, auto ISSUE, auto SCALES, auto WAIT, uint32_t (&tb)[C::FN], uint32_t (&tnb)[C::FN]) {
          constexpr bool kIssue = decltype(ISSUE)::value;
          constexpr bool kScales = decltype(SCALES)::value;
          constexpr int kWait = decltype(WAIT)::value;
          half(0, bqc, afc, tb, [&](int i) {
#pragma unroll
            for (int r = R1 * i; r < R1 * i + R1; ++r)
              if (r < NR) read_frag(s, 1, r, bqn, afn);
          });
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) asm volatile("" : "+a"(acc[fm][fn]));
          if constexpr (kWait >= 0) {
            wait_lgkm0();
            wait_vm<kWait>();
            stage_barrier();
          }
          __builtin_amdgcn_sched_barrier(0);
          half(1, bqn, afn, tb, [&](int i) {
            if constexpr (kWait >= 0) {
#pragma unroll
              for (int r = R2 * i; r < R2 * i + R2; ++r) {
                if (r < NS) read_scale(s + 1, r, tnb);
                else if (r < NS + NR) read_frag(s + 1, 0, r - NS, bqc, afc);
              }
            }
            if constexpr (kIssue) {
#pragma unroll
              for (int j = D2 * i; j < D2 * i + D2; ++j) {
                if (j < C::LOADS) issue_one(s + 3, j);
                if (kScales && j == C::LOADS - 1) issue_scales((s + 3) >> 2);
              }
            }
          });
        };
        using T = std::integral_constant<bool, true>;
        using F = std::integral_constant<bool, false>;
        using WL = std::integral_constant<int, C::LOADS>;
        wait_vm<2 * C::LOADS>();
        stage_barrier();
#pragma unroll
        for (int r = 0; r < NS; ++r) read_scale(0, r, sb);
#pragma unroll
        for (int r = 0; r < NR; ++r) read_frag(0, 0, r, bqc, afc);
        int s = 0;
        for (; s + 4 < nst; s += 4) {
          step(s, T{}, F{}, WL{}, sb, nb);
          step(s + 1, T{}, T{}, WL{}, nb, sb);
          step(s + 2, T{}, F{}, WL{}, sb, nb);
          step(s + 3, T{}, F{}, WL{}, nb, sb);
        }
        step(s, T{}, F{}, WL{}, sb, nb);
        step(s + 1, F{}, F{}, WL{}, nb, sb);
        step(s + 2, F{}, F{}, std::integral_constant<int, 0>{}, sb, nb);
        step(s + 3, F{}, F{}, std::integral_constant<int, -1>{}, nb, sb);
      };
      if constexpr (C::WAVES_M == 1 && C::FM == 4) {
        // the full 128-row tile: a unit of at most 96 rows leaves its last fragment empty
        if (mrows > 96) bf16_kloop(std::integral_constant<int, 4>{});
        else bf16_kloop(std::integral_constant<int, 3>{});
      } else {
        bf16_kloop(std::integral_constant<int, C::FM>{});
      }
    }


    // ---- between units ----
    clock.lap(0);
    stage_barrier();   // every wave is done reading the stage and scale buffers
    const int e_row0 = row0, e_mrows = mrows, e_nt = nt;
    const int un = __builtin_amdgcn_readfirstlane(next());
    clock.lap(1);
    // the next unit's set-up and first PF stages: issued once the accumulators
    // are dead (after the last staging write; before a direct epilogue), so that
    // its offsets need no registers beside them
    auto prefetch = [&]() {
      if (EC::EARLY && un >= 0) {
        setup(un);
        issue_scales(0);
#pragma unroll
        for (int s = 0; s < EC::PF; ++s) issue(s);
      }
    };
    if constexpr (!EC::STAGED) prefetch();

    // ---- epilogue: registers -> C in permuted row order ----
    // The products take the weights as their first operand, so each
    // fragment's accumulator is the transposed 32x32 tile: lane l holds tile
    // row l % 32 and its accumulator q holds column 8*(q/4) + 4*(l/32) + q%4
    // of the fragment's 32-column block (four runs of four consecutive
    // columns; the other four runs sit in the partner lane l ^ 32).  SwiGLU:
    // fragment fh holds the gate columns of 32-column block 2fh, fragment
    // fh + FN/2 the matching up columns of block 2fh + 1 (see frag_block), so
    // gate and up of an output column share a lane and an accumulator index.
    {
      // the epilogue's lane-derived values come from a fresh lane index
      const int lane = lane_id();
      const int tid = wave * 64 + lane;
      const int wm0 = (wave / C::WAVES_N) * C::WM;
      const int wn0 = (wave % C::WAVES_N) * C::WN;
      const int l32 = lane & 31;
      const int g = lane >> 5;
      // rows this unit stores (none for a unit run only to keep a block's halves in step)
      const int srows = store ? e_mrows : 0;
      constexpr int HF = C::FN / 2;
      const int ld = EPI == 0 ? p.N : p.n_out;
      const int col0 = e_nt * EC::TC;               // the tile's first output column
      const int ncols = min(EC::TC, ld - col0);     // a multiple of 32 (N and n_out are)
      if constexpr (!EC::STAGED) {
        // fp32: each run of four columns straight from the accumulators
        const bool vec = (reinterpret_cast<uintptr_t>(p.c) & 15) == 0;
        auto store4 = [&](size_t o, float v0, float v1, float v2, float v3) {
          float* const d = static_cast<float*>(p.c) + o;
          if (vec) {
            *reinterpret_cast<float4*>(d) = make_float4(v0, v1, v2, v3);
          } else {
            d[0] = v0; d[1] = v1; d[2] = v2; d[3] = v3;
          }
        };
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          const int r = wm0 + fm * 32 + l32;
          const size_t orow = (size_t)(e_row0 + r) * ld;
          if constexpr (EPI == 0) {
#pragma unroll
            for (int f = 0; f < C::FN; ++f) {
              const int n0 = col0 + wn0 + frag_block(f) * 32;
              if (r < srows && n0 < ld) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  store4(orow + n0 + 8 * j + 4 * g, acc[fm][f][4 * j], acc[fm][f][4 * j + 1],
                         acc[fm][f][4 * j + 2], acc[fm][f][4 * j + 3]);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int fh = 0; fh < HF; ++fh) {
              const int i0 = col0 + (wave % C::WAVES_N) * (C::WN / 2) + fh * 32;
              if (r < srows && i0 < ld) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  float a[4];
#pragma unroll
                  for (int t = 0; t < 4; ++t) a[t] = silu_mul(acc[fm][fh][4 * j + t], acc[fm][fh + HF][4 * j + t]);
                  store4(orow + i0 + 8 * j + 4 * g, a[0], a[1], a[2], a[3]);
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      } else {
        constexpr bool MX = EC::MX;
        static_assert(!MX || EPI != 0, "MXFP8 output needs the SwiGLU epilogue");
#pragma unroll
        for (int pass = 0; pass < EC::PASSES; ++pass) {
          const int pr0 = pass * EC::PROWS;   // first tile row of the pass
          if (wm0 >= pr0 && wm0 < pr0 + EC::PROWS) {   // this wave's rows belong to the pass
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
              uint8_t* const srow = lds + EC::BASE + (wm0 - pr0 + fm * 32 + l32) * EC::PITCH;   // this lane's staged row
              if constexpr (EPI == 0) {
#pragma unroll
                for (int f = 0; f < C::FN; ++f) {
                  uint8_t* const d = srow + (wn0 + frag_block(f) * 32 + 4 * g) * 2;
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    // v_cvt_pk_bf16_f32 (RNE)
                    const uint32_t h0 = __builtin_bit_cast(uint16_t, (__bf16)acc[fm][f][4 * j]);
                    const uint32_t h1 = __builtin_bit_cast(uint16_t, (__bf16)acc[fm][f][4 * j + 1]);
                    const uint32_t h2 = __builtin_bit_cast(uint16_t, (__bf16)acc[fm][f][4 * j + 2]);
                    const uint32_t h3 = __builtin_bit_cast(uint16_t, (__bf16)acc[fm][f][4 * j + 3]);
                    *reinterpret_cast<uint2*>(d + 16 * j) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                  }
                  __builtin_amdgcn_sched_barrier(0);
                }
              } else {
#pragma unroll
                for (int fh = 0; fh < HF; ++fh) {
                  const int lc = (wave % C::WAVES_N) * (C::WN / 2) + fh * 32;   // the block's first tile column
                  float a[16];
#pragma unroll
                  for (int q = 0; q < 16; ++q) a[q] = silu_mul(acc[fm][fh][q], acc[fm][fh + HF][q]);
                  if constexpr (MX) {
                    // one 32-element MX block per row: this lane's 16 values and its partner's
                    float amax = 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(a[q]));
                    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
                    const int x = mxfp8_block_exp(amax);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                      *reinterpret_cast<uint32_t*>(srow + lc + 8 * j + 4 * g) =
                          e4m3x4_rne(ldexpf(a[4 * j], -x), ldexpf(a[4 * j + 1], -x), ldexpf(a[4 * j + 2], -x),
                                     ldexpf(a[4 * j + 3], -x));
                    if (g == 0) lds[EC::BASE + EC::SC_OFF + (wm0 - pr0 + fm * 32 + l32) * (EC::TC / 32) + lc / 32] = (uint8_t)(x + 127);
                  } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                      const uint32_t h0 = __builtin_bit_cast(uint16_t, (__bf16)a[4 * j]);
                      const uint32_t h1 = __builtin_bit_cast(uint16_t, (__bf16)a[4 * j + 1]);
                      const uint32_t h2 = __builtin_bit_cast(uint16_t, (__bf16)a[4 * j + 2]);
                      const uint32_t h3 = __builtin_bit_cast(uint16_t, (__bf16)a[4 * j + 3]);
                      *reinterpret_cast<uint2*>(srow + (lc + 8 * j + 4 * g) * 2) =
                          make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                    }
                  }
                  __builtin_amdgcn_sched_barrier(0);
                }
              }
            }
          }
          if (pass == EC::PASSES - 1) {
            clock.lap(2);
            prefetch();
          }
          stage_barrier();
          if (pass == EC::PASSES - 1) clock.lap(3);
          // The pass's rows -> C in whole row segments, 16 bytes a thread.  The
          // staging is read with lds_read16/lds_read4 (see there): a plain LDS
          // read here would be ordered after the next unit's DMA just issued.
          const int prows = min(EC::PROWS, srows - pr0);   // may be <= 0
          constexpr int CB = MX ? 16 : 8;                  // elements per 16-byte chunk
          constexpr int CPR = EC::TC / CB;                 // chunks per staged row
          const uint32_t sbase = lds_addr(lds) + EC::BASE;
          if constexpr (!MX) {
            const bool vec = ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0) && (ld % 8 == 0);
            uint16_t* const out = static_cast<uint16_t*>(p.c) + (size_t)(e_row0 + pr0) * ld + col0;
            for (int idx = tid; idx < prows * CPR; idx += C::NT) {
              const int r = idx / CPR, c = (idx % CPR) * CB;
              if (c >= ncols) continue;
              const uint4 v = lds_read16(sbase + r * EC::PITCH + c * 2);
              uint16_t* dst = out + (size_t)r * ld + c;
              if (vec) {
                *reinterpret_cast<uint4*>(dst) = v;
              } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
              }
            }
          } else {
            const bool vec = (reinterpret_cast<uintptr_t>(p.c) & 15) == 0;   // ld % 32 == 0 (the host checks)
            uint8_t* const out = static_cast<uint8_t*>(p.c) + (size_t)(e_row0 + pr0) * ld + col0;
            for (int idx = tid; idx < prows * CPR; idx += C::NT) {
              const int r = idx / CPR, c = (idx % CPR) * CB;
              if (c >= ncols) continue;
              const uint4 v = lds_read16(sbase + r * EC::PITCH + c);
              uint8_t* dst = out + (size_t)r * ld + c;
              if (vec) {
                *reinterpret_cast<uint4*>(dst) = v;
              } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 16; ++j) dst[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
              }
            }
            // the rows' E8M0 bytes: TC / 32 = 4 consecutive bytes per row
            static_assert(EC::TC / 32 == 4, "one 4-byte word of scales per staged row");
            const int sld = ld / 32;
            const bool svec = (reinterpret_cast<uintptr_t>(p.c_scales) & 3) == 0 && sld % 4 == 0 && ncols == EC::TC;
            for (int idx = tid; idx < prows; idx += C::NT) {
              const uint32_t w = lds_read4(sbase + EC::SC_OFF + idx * 4);
              uint8_t* const osc = p.c_scales + (size_t)(e_row0 + pr0 + idx) * sld + col0 / 32;
              if (svec) {
                *reinterpret_cast<uint32_t*>(osc) = w;
              } else {
                for (int b = 0; b < ncols / 32; ++b) osc[b] = (uint8_t)(w >> (8 * b));
              }
            }
          }
          if (pass == EC::PASSES - 1) clock.lap(4);
          stage_barrier();   // the staging is read before anything writes it again
          if (pass == EC::PASSES - 1) clock.lap(5);
        }
      }
    }
    settle();
    if (un < 0) {
      clock.lap(6);
      break;
    }
    if constexpr (!EC::EARLY) {
      setup(un);
      issue_scales(0);
    }
    // the next unit's stages that the staging's buffers hold (all of them
    // without the early start)
#pragma unroll
    for (int s = EC::EARLY ? EC::PF : 0; s < C::NST; ++s) issue(s);
    clock.lap(6);
  }
  clock.flush(BM == 32 ? 0 : BM == 64 ? 1 : BM == 128 ? 2 : 3, tid_in == 0 && store);
}

template <int BM, bool FP8, int EPI, int OUT, bool TILED>
__global__ __launch_bounds__((64 * dma_waves<BM, FP8, EPI>())) void gemm_dma_kernel(Params p) {
  using C = Cfg2<BM, FP8, dma_waves<BM, FP8, EPI>()>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_TOTAL];

  const int count = *p.tile_count;
  const int units = count * p.n_tiles;
  if (units == 0) return;   // a class no expert fills (the same in every thread)
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = (units + kXcds - 1) / kXcds;

  // Units of an XCD's range are handed out dynamically (blocks whose units
  // end early take more; blocks that start late take fewer).  Thread 0 draws
  // the next index with an atomic one unit ahead; the index reaches the other
  // threads through a slot in scale buffer 1, which is idle between a unit's
  // last products and the next unit's second stage.  A block drains its own
  // XCD's range first, then (the end game) the other XCDs' ranges that still
  // held units when thread 0 read their counters after its own range (a
  // counter only grows: a stale read can only add a visit that draws nothing).
  // With fewer than two units per block (decode at T <= 2) every range is
  // drawn out by the blocks' first draws, and the end game is skipped.
  int* const slot = reinterpret_cast<int*>(lds + C::NST * C::LDS_STAGE + C::LDS_SG);
  const int rounds = units >= 2 * (int)gridDim.x ? kXcds : 1;
  uint32_t open = 0;   // bit x: XCD x's range had units left
  for (int k = 0; k < rounds; ++k) {
    const int x = (xcd + k) % kXcds;   // the XCD whose range this round drains
    if (k == 1) {
      if (threadIdx.x == 0) {
        uint32_t m = 0;
        for (int y = 0; y < kXcds; ++y)
          if (p.unit_ctr[y] < min(units, (y + 1) * per_xcd) - y * per_xcd) m |= 1u << y;
        slot[1] = (int)m;
      }
      stage_barrier();
      open = (uint32_t)__builtin_amdgcn_readfirstlane(slot[1]);
      stage_barrier();   // read before any unit's LDS use
    }
    if (k > 0 && !((open >> x) & 1u)) continue;
    const int u_first = x * per_xcd;
    const int u_end = min(units, u_first + per_xcd);
    if (threadIdx.x == 0) slot[0] = atomicAdd(&p.unit_ctr[x], 1);
    stage_barrier();
    const int u = u_first + slot[0];
    stage_barrier();   // the slot is read before it is written again
    if (u >= u_end) continue;   // the same in every thread
    // Thread 0's draw of the unit after the current one, in a scalar register
    // (wave 0's first lane is thread 0).  next() publishes it and issues the
    // following draw; settle() takes that draw's result after the epilogue, so
    // that the atomic's latency passes under it.
    int d = 0;
    if (threadIdx.x == 0) d = atomicAdd(&p.unit_ctr[x], 1);
    int drawn = __builtin_amdgcn_readfirstlane(d);
    auto next = [&]() -> int {
      if (threadIdx.x == 0) slot[0] = drawn;
      stage_barrier();
      const int n = u_first + slot[0];
      d = 0;
      if (threadIdx.x == 0 && n < u_end) d = atomicAdd(&p.unit_ctr[x], 1);
      return n < u_end ? n : -1;
    };
    auto settle = [&]() { drawn = __builtin_amdgcn_readfirstlane(d); };
    run_units<BM, FP8, EPI, OUT, TILED, C::NW>(p, u, count, threadIdx.x, lds, true, next, settle);
    stage_barrier();   // every wave is done with the LDS and the slots
  }
}

// ---- every row-tile class of a call in one launch ------------------------
//
// The full 256-row tiles are bound by the matrix cores; the <= 32-row tiles
// (the remainders of experts with few rows: the tail of a skewed routing)
// only stream their experts' weights, and the 64- and 128-row tiles sit in
// between.  Run one class after another, the weight stream runs with the
// matrix cores idle; and one block streams at most some tens of GB/s (its
// three-stage ring keeps two stages in flight: about 27 GB/s per <= 32-row
// unit beside the full tiles), so that stream needs many CUs at once.  Here every CU runs one block of eight waves that
// works through the classes' unit queues in turn: kSmallCus blocks per XCD
// take the <= 32-row units first (two at a time: waves 0-3 and 4-7 each run
// one unit in their own half of the LDS), then the 64-, 128- and 256-row
// ones; the other blocks take them in the opposite order.  The weight stream
// of the small units then runs under the matrix-core work of the other CUs,
// and every block stays busy until the last queue is empty.  Both halves of
// a block run the same barriers: a half without a unit of its own runs its
// partner's unit without storing it.  Units are drawn per XCD from the
// planner's lists as the single-class launches draw them (one unit ahead), so
// every output row is written once, by the same per-unit code.
constexpr int kSmallHalfLds = 81920;   // LDS of one half running a <= 32-row unit
constexpr int kSmallCus = 4;           // blocks per XCD that start on the <= 32-row units

template <bool FP8, int EPI, int OUT>
__global__ __launch_bounds__(512) void gemm_mixed_kernel(Params p, int small_cus) {
  using CF = Cfg2<256, FP8, 8>;
  using CS = Cfg2<32, FP8, 4>;
  static_assert(CS::LDS_TOTAL <= kSmallHalfLds, "a <= 32-row unit fits half the LDS");
  constexpr int kSlots = CF::NST * CF::LDS_STAGE + CF::LDS_SG;   // scale buffer 1 of the 256-row units
  static_assert(kSmallHalfLds + CS::LDS_TOTAL <= kSlots && Cfg2<128, FP8, 8>::LDS_TOTAL <= kSlots,
                "the draw slots lie beyond the LDS of every unit but the 256-row ones");
  static_assert(kSlots + 3 * sizeof(int) <= CF::LDS_TOTAL, "three slots inside the LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS_TOTAL];
  int* const slot = reinterpret_cast<int*>(lds + kSlots);   // this block's next draw, per half; [2]: the end game's queues

  const int xcd = blockIdx.x % kXcds;
  const bool small_first = blockIdx.x / kXcds < small_cus;
  const int half = threadIdx.x >> 8;
  const Tile* const lists = p.tiles;
  const int32_t* const counts = p.tile_count;
  int32_t* const ctr = p.unit_ctr;
  auto none = []() -> int { return -1; };

  // The block drains its own XCD's queues first, then (the end game) those of
  // the other XCDs in turn: the XCDs do not finish their ranges together
  // (prefill896 FC1: their last blocks ended up to 0.36 ms apart), and a
  // block whose XCD is done adds its matrix cores to a late XCD's work.  For
  // the end game thread 0 reads every queue's counter once and the block
  // visits only the queues that still held units then (a counter only grows,
  // so a stale read can only add a visit that draws nothing).
  uint32_t open = 0;   // bit c * kXcds + x: queue (class c, XCD x) had units left
  for (int k = 0; k < kXcds; ++k) {
    const int x = (xcd + k) % kXcds;   // the XCD whose queues this round drains
    if (k == 1) {
      if (threadIdx.x == 0) {
        uint32_t m = 0;
        for (int c = 0; c < kClasses; ++c) {
          const int units = counts[c] * p.n_tiles;
          const int per_xcd = (units + kXcds - 1) / kXcds;
          for (int y = 0; y < kXcds; ++y)
            if (ctr[c * kXcds + y] < min(units, (y + 1) * per_xcd) - y * per_xcd) m |= 1u << (c * kXcds + y);
        }
        slot[2] = (int)m;
      }
      stage_barrier();
      open = (uint32_t)__builtin_amdgcn_readfirstlane(slot[2]);
      stage_barrier();   // read before any unit's LDS use
    }
    int ph = 0;          // position in this block's queue order
    bool have = false;   // <= 32-row queue: the slots already hold the next draws
    while (ph < kClasses) {
      const int c = small_first ? ph : kClasses - 1 - ph;   // row-tile class of the current queue
      if (k > 0 && !((open >> (c * kXcds + x)) & 1u)) {
        ++ph;
        continue;
      }
      const int cnt = counts[c];
      const int units = cnt * p.n_tiles;
      const int per_xcd = (units + kXcds - 1) / kXcds;
      const int u0 = x * per_xcd, u1 = min(units, u0 + per_xcd);
      int32_t* const uc = ctr + c * kXcds + x;
      Params q = p;
      q.tiles = lists + c * p.tile_cap;
      if (c == 0) {
        // two units side by side, one per half, each drawn by the half's first thread
        const bool drawer = (threadIdx.x & 255) == 0;
        if (!have && drawer) slot[half] = atomicAdd(uc, 1);
        stage_barrier();
        const int a = u0 + slot[0], b = u0 + slot[1];
        stage_barrier();   // both slots read before either is written again
        const bool va = a < u1, vb = b < u1;
        if (!va && !vb) {
          ++ph;
          have = false;
          continue;
        }
        int nxt = 0;
        if (drawer) nxt = atomicAdd(uc, 1);   // one unit ahead
        const bool mine = half ? vb : va;
        const int u = (half ? vb : !va) ? b : a;   // a half without a unit runs its partner's
        run_units<32, FP8, EPI, OUT, true, 4>(q, u, cnt, threadIdx.x & 255, lds + half * kSmallHalfLds, mine, none,
                                              [] {});
        stage_barrier();   // every wave is done with the LDS
        if (drawer) slot[half] = nxt;
        have = true;
        continue;
      }
      // one unit stream for the whole block, the next unit's first stages under each epilogue
      if (threadIdx.x == 0) slot[0] = atomicAdd(uc, 1);
      stage_barrier();
      const int a = u0 + slot[0];
      stage_barrier();   // the slot is read before it is written again
      if (a < u1) {
        // thread 0's draws, one unit ahead, as in gemm_dma_kernel
        int d = 0;
        if (threadIdx.x == 0) d = atomicAdd(uc, 1);
        int drawn = __builtin_amdgcn_readfirstlane(d);
        auto next = [&]() -> int {
          if (threadIdx.x == 0) slot[0] = drawn;
          stage_barrier();
          const int n = u0 + slot[0];
          d = 0;
          if (threadIdx.x == 0 && n < u1) d = atomicAdd(uc, 1);
          return n < u1 ? n : -1;
        };
        auto settle = [&]() { drawn = __builtin_amdgcn_readfirstlane(d); };
        if (c == 3) run_units<256, FP8, EPI, OUT, true, 8>(q, a, cnt, threadIdx.x, lds, true, next, settle);
        else if (c == 2) run_units<128, FP8, EPI, OUT, true, 8>(q, a, cnt, threadIdx.x, lds, true, next, settle);
        else run_units<64, FP8, EPI, OUT, true, 8>(q, a, cnt, threadIdx.x, lds, true, next, settle);
        stage_barrier();   // every wave is done with the LDS and the slot
      }
      have = false;
      ++ph;
    }
  }
}

// ---- load-time weight tiling ------------------------------------------
//
// Tiled order of one weight matrix (kept instead of the canonical one): for
// expert e, n-tile nt and 128-element stage s, the 16 KB block at
// ((e * n_tiles + nt) * nst + s) * 16384 holds at byte q exactly what the DMA
// kernels' B load puts at byte q of the stage's LDS B area (line q / 128 =
// tile columns 2*line, 2*line + 1; slot (q % 128) / 16 XOR the line swizzle
// -> column 2*line + slot' / 4, 16-byte chunk slot' % 4 of its 64 stage
// bytes).  Scales: for scale group g (512 K elements) the 4 KB block at
// ((e * n_tiles + nt) * (K / 512) + g) * 4096 holds at byte 16c + b scale
// byte 16g + b of tile column c's row.  Needs K % 512 == 0 and N % 256 == 0,
// so every tile column is one distinct weight row and the map is a bijection.

// canonical row r -> (n-tile, tile column): the inverse of w_row_of<kSwiGroup>
__device__ inline void tile_col_of(int layout, int r, int n_out, int& nt, int& j) {
  if (layout == 0) {
    nt = r / kBN;
    j = r % kBN;
    return;
  }
  const int up = layout == 1 ? (r >= n_out ? 1 : 0) : (r & 1);
  const int i = layout == 1 ? r - up * n_out : r >> 1;
  nt = i / (kBN / 2);
  const int ii = i % (kBN / 2);
  j = (ii / 32) * kSwiGroup + up * 32 + ii % 32;
}

// one thread per 16-byte chunk of the canonical packed matrix
template <bool TO_TILED>
__global__ __launch_bounds__(256) void tile_packed_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int E, int N, int K, int layout) {
  const int cpr = K / 32;   // 16-byte chunks per row (K/2 bytes)
  const int64_t total = (int64_t)E * N * cpr;
  const int n_tiles = N / kBN, nst = K / 128;
  const int n_out = layout == 0 ? N : N / 2;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total; id += (int64_t)gridDim.x * 256) {
    const int c = (int)(id % cpr);
    const int64_t er = id / cpr;
    const int r = (int)(er % N);
    const int e = (int)(er / N);
    int nt, j;
    tile_col_of(layout, r, n_out, nt, j);
    const int line = j >> 1;
    const int slot = ((j & 1) * 4 + (c & 3)) ^ b_swz(line);
    const int64_t t = (((int64_t)e * n_tiles + nt) * nst + (c >> 2)) * 16384 + line * 128 + slot * 16;
    const int64_t cp = er * (K / 2) + (int64_t)c * 16;
    if (TO_TILED) *reinterpret_cast<uint4*>(dst + t) = *reinterpret_cast<const uint4*>(src + cp);
    else *reinterpret_cast<uint4*>(dst + cp) = *reinterpret_cast<const uint4*>(src + t);
  }
}

// one thread per 16-byte scale group of a canonical row
template <bool TO_TILED>
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int E, int N, int K, int layout) {
  const int gpr = K / 512;
  const int64_t total = (int64_t)E * N * gpr;
  const int n_tiles = N / kBN;
  const int n_out = layout == 0 ? N : N / 2;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total; id += (int64_t)gridDim.x * 256) {
    const int g = (int)(id % gpr);
    const int64_t er = id / gpr;
    const int r = (int)(er % N);
    const int e = (int)(er / N);
    int nt, j;
    tile_col_of(layout, r, n_out, nt, j);
    const int64_t t = (((int64_t)e * n_tiles + nt) * gpr + g) * 4096 + j * 16;
    const int64_t cp = er * (K / 32) + (int64_t)g * 16;
    if (TO_TILED) *reinterpret_cast<uint4*>(dst + t) = *reinterpret_cast<const uint4*>(src + cp);
    else *reinterpret_cast<uint4*>(dst + cp) = *reinterpret_cast<const uint4*>(src + t);
  }
}

// ---- planning: expert offsets -> per-class tile lists ------------------

__device__ inline int4 wave_incl_scan4(int4 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int4 o;
    o.x = __shfl_up(v.x, off, 64);
    o.y = __shfl_up(v.y, off, 64);
    o.z = __shfl_up(v.z, off, 64);
    o.w = __shfl_up(v.w, off, 64);
    if (lane >= off) { v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w; }
  }
  return v;
}

// Full tiles have `big` rows (256 or 128) and go to class 3 or 2; an expert's
// remainder goes to the smallest class of 32/64/128/256 rows that holds it.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                    int big_log2, Tile* __restrict__ lists, int cap,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ unit_ctr) {
  if (threadIdx.x < kClasses * kXcds) unit_ctr[threadIdx.x] = 0;
  __shared__ int4 wave_tot[16];
  __shared__ int4 carry;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = make_int4(0, 0, 0, 0);
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int n = 0, start = 0;
    if (e < E) {
      start = offsets[e];
      n = offsets[e + 1] - start;
    }
    const int big = 1 << big_log2;
    const int full = n >> big_log2, rem = n & (big - 1);
    const int cls = rem == 0 ? -1 : rem <= 32 ? 0 : rem <= 64 ? 1 : rem <= 128 ? 2 : 3;
    const int full_cls = big_log2 == 8 ? 3 : 2;
    int4 c = make_int4(cls == 0, cls == 1, (cls == 2) + (full_cls == 2 ? full : 0),
                       (cls == 3) + (full_cls == 3 ? full : 0));
    int4 incl = wave_incl_scan4(c);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      int4 t = lane < 16 ? wave_tot[lane] : make_int4(0, 0, 0, 0);
      t = wave_incl_scan4(t);
      if (lane < 16) wave_tot[lane] = t;
    }
    __syncthreads();
    if (wid > 0) {
      const int4 b = wave_tot[wid - 1];
      incl.x += b.x; incl.y += b.y; incl.z += b.z; incl.w += b.w;
    }
    const int4 cb = carry;
    const int p0 = cb.x + incl.x - c.x, p1 = cb.y + incl.y - c.y;
    const int p2 = cb.z + incl.z - c.z, p3 = cb.w + incl.w - c.w;
    // full tiles first, then the remainder, so an expert's tiles are in row order
    const int pf = full_cls == 3 ? p3 : p2;
    for (int q = 0; q < full; ++q) lists[full_cls * cap + pf + q] = Tile{e, start + big * q};
    const int rs = start + big * full;
    if (cls == 3) lists[3 * cap + p3 + (full_cls == 3 ? full : 0)] = Tile{e, rs};
    if (cls == 2) lists[2 * cap + p2 + (full_cls == 2 ? full : 0)] = Tile{e, rs};
    if (cls == 1) lists[1 * cap + p1] = Tile{e, rs};
    if (cls == 0) lists[0 * cap + p0] = Tile{e, rs};
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry = make_int4(cb.x + incl.x, cb.y + incl.y, cb.z + incl.z, cb.w + incl.w);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[0] = carry.x;
    counts[1] = carry.y;
    counts[2] = carry.z;
    counts[3] = carry.w;
  }
}

int list_capacity(int rows, int E) { return rows / 32 + E + 8; }  // >= rows/128 + E per class

template <typename KernelT>
int persistent_grid(KernelT kernel, int threads = kThreads) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = num_cus() * per_cu;
  return (grid + kXcds - 1) / kXcds * kXcds;
}

// PATH: 0 register-staged kernels, 1 DMA kernels on canonical weights, 2 DMA
// kernels on tiled weights
template <int BM, bool FP8, int EPI, int OUT, int PATH>
int class_grid() {
  static int grid = 0;  // per instantiation; one device type (gfx950)
  if (grid == 0) {
    if constexpr (PATH != 0)
      grid = persistent_grid(gemm_dma_kernel<BM, FP8, EPI, OUT, PATH == 2>, 64 * dma_waves<BM, FP8, EPI>());
    else grid = persistent_grid(gemm_kernel<BM, FP8, EPI, OUT>);
  }
  return grid;
}

// `reserve`: CUs per XCD left without a block of this launch, so that a
// kernel on another stream (the routed expert copy) finds a free CU beside a
// persistent GEMM that otherwise fills every CU's LDS.
template <int BM, bool FP8, int EPI, int OUT, int PATH>
moe_status launch_class(const Params& p, hipStream_t s, int reserve) {
  int grid = class_grid<BM, FP8, EPI, OUT, PATH>();
  if (reserve > 0) {
    const int per_cu = grid / num_cus() > 0 ? grid / num_cus() : 1;
    grid = (grid - reserve * kXcds * per_cu) / kXcds * kXcds;
    if (grid < kXcds) grid = kXcds;
  }
  if constexpr (PATH != 0)
    hipLaunchKernelGGL((gemm_dma_kernel<BM, FP8, EPI, OUT, PATH == 2>), dim3(grid),
                       dim3(64 * dma_waves<BM, FP8, EPI>()), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, FP8, EPI, OUT>), dim3(grid), dim3(kThreads), 0, s, p);
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

// One launch per row-tile class, in order, on the caller's stream.  (Running
// the HBM-bound small-tile classes beside the full-tile class on a slice of
// the CUs was measured slower: a few CUs cannot pull the weight stream at
// HBM rate, and the full tiles lose those CUs for longer.)
// Fewest rows an expert needs for a tile of each class (the planner's rule:
// remainders of 1-32, 33-64, 65-128, 129-256 rows; full 128- or 256-row tiles
// need at least that many).  A class whose minimum exceeds every expert's row
// count gets no tiles and is not launched.
constexpr int kClassMinRows[kClasses] = {1, 33, 65, 129};

template <bool FP8, int EPI, int OUT, int PATH>
moe_status launch_all(Params p, const Tile* lists, int cap, const int32_t* counts, hipStream_t s,
                      int reserve, int max_rows) {
  int32_t* const ctr = p.unit_ctr;
  auto at = [&](int c) {
    p.tiles = lists + c * cap;
    p.tile_count = counts + c;
    p.unit_ctr = ctr + c * kXcds;
  };
  if constexpr (FP8 && PATH == 2) {
    // every class in one launch when the full 256-row class can have tiles
    if (reserve == 0 && max_rows >= kClassMinRows[3]) {
      Params q = p;
      q.tiles = lists;
      q.tile_cap = cap;
      q.tile_count = counts;
      q.unit_ctr = ctr;
      hipLaunchKernelGGL((gemm_mixed_kernel<FP8, EPI, OUT>), dim3(num_cus() / kXcds * kXcds), dim3(512), 0, s,
                         q, kSmallCus);
      MXMOE_HIP(hipGetLastError());
      return MOE_OK;
    }
  }
  at(0); MXMOE_TRY((launch_class<32, FP8, EPI, OUT, PATH>(p, s, reserve)));
  if (max_rows < kClassMinRows[1]) return MOE_OK;
  at(1); MXMOE_TRY((launch_class<64, FP8, EPI, OUT, PATH>(p, s, reserve)));
  if (max_rows < kClassMinRows[2]) return MOE_OK;
  at(2); MXMOE_TRY((launch_class<128, FP8, EPI, OUT, PATH>(p, s, reserve)));
  if (max_rows < kClassMinRows[3]) return MOE_OK;
  // the bf16 DMA kernel's full tile is 128 rows (its 256-row stages do not fit
  // in LDS), so its class-3 list is empty
  if constexpr (!(PATH != 0 && !FP8)) {
    at(3); MXMOE_TRY((launch_class<256, FP8, EPI, OUT, PATH>(p, s, reserve)));
  }
  return MOE_OK;
}

template <bool FP8, int EPI, int PATH>
moe_status dispatch_out(const Params& p, int c_dtype, const Tile* lists, int cap,
                        const int32_t* counts, hipStream_t s, int reserve, int max_rows) {
  if (c_dtype == MOE_OUT_FP32)
    return launch_all<FP8, EPI, MOE_OUT_FP32, PATH>(p, lists, cap, counts, s, reserve, max_rows);
  if (c_dtype == MOE_OUT_BF16)
    return launch_all<FP8, EPI, MOE_OUT_BF16, PATH>(p, lists, cap, counts, s, reserve, max_rows);
  if constexpr (PATH != 0 && EPI != 0)
    return launch_all<FP8, EPI, MOE_OUT_MXFP8_E4M3, PATH>(p, lists, cap, counts, s, reserve, max_rows);
  return fail(MOE_ERR_NOT_IMPLEMENTED,
              "grouped GEMM: MXFP8 output needs the SwiGLU epilogue and K %% 512 == 0");
}

template <bool FP8, int PATH>
moe_status dispatch_epi(const Params& p, int epi, int c_dtype, const Tile* lists, int cap,
                        const int32_t* counts, hipStream_t s, int reserve, int max_rows) {
  if (epi == MOE_EPI_NONE) return dispatch_out<FP8, 0, PATH>(p, c_dtype, lists, cap, counts, s, reserve, max_rows);
  return dispatch_out<FP8, 1, PATH>(p, c_dtype, lists, cap, counts, s, reserve, max_rows);
}

template <bool FP8>
moe_status dispatch_path(int path, const Params& p, int epi, int c_dtype, const Tile* lists, int cap,
                         const int32_t* counts, hipStream_t s, int reserve, int max_rows) {
  if (path == 2) return dispatch_epi<FP8, 2>(p, epi, c_dtype, lists, cap, counts, s, reserve, max_rows);
  if (path == 1) return dispatch_epi<FP8, 1>(p, epi, c_dtype, lists, cap, counts, s, reserve, max_rows);
  return dispatch_epi<FP8, 0>(p, epi, c_dtype, lists, cap, counts, s, reserve, max_rows);
}

}  // namespace

size_t gemm_ws_bytes(int rows, int E) {
  const size_t cap = (size_t)list_capacity(rows, E);
  return align_up(kClasses * cap * sizeof(Tile), 256) + 256;
}

moe_status validate_gemm(const moe_gemm_args& a) {
  if (!a.a || !a.w_packed || !a.w_scales || !a.expert_offsets || !a.c)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: a, w_packed, w_scales, expert_offsets and c are required");
  if (a.a_dtype != MOE_ACT_BF16 && a.a_dtype != MOE_ACT_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: bad a_dtype %d", a.a_dtype);
  if (a.a_dtype == MOE_ACT_MXFP8_E4M3 && !a.a_scales)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: MXFP8 A needs a_scales");
  if (a.epilogue < MOE_EPI_NONE || a.epilogue > MOE_EPI_SWIGLU_INTERLEAVED)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: bad epilogue %d", a.epilogue);
  if (a.c_dtype < MOE_OUT_FP32 || a.c_dtype > MOE_OUT_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: bad c_dtype %d", a.c_dtype);
  if (a.rows < 0 || a.E < 1 || a.N < 1 || a.K < 1 || a.a_rows < 0 || a.a_gather_div < 1)
    return fail(MOE_ERR_SHAPE, "grouped GEMM: rows %d, E %d, N %d, K %d, a_rows %d, div %d out of range",
                a.rows, a.E, a.N, a.K, a.a_rows, a.a_gather_div);
  if (a.K % 32 || a.N % 32)
    return fail(MOE_ERR_SHAPE, "grouped GEMM: K (%d) and N (%d) must be multiples of 32", a.K, a.N);
  if (a.epilogue != MOE_EPI_NONE && a.N % 64)
    return fail(MOE_ERR_SHAPE, "grouped GEMM: a SwiGLU epilogue needs N %% 64 == 0 (gate + up), got %d", a.N);
  if (a.c_dtype == MOE_OUT_MXFP8_E4M3) {
    if (a.epilogue == MOE_EPI_NONE || a.K % 512)
      return fail(MOE_ERR_NOT_IMPLEMENTED,
                  "grouped GEMM: MXFP8 output needs the SwiGLU epilogue and K %% 512 == 0 (K = %d)", a.K);
    if (!a.c_scales) return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: MXFP8 output needs c_scales");
  }
  if (a.K % 512 == 0) {
    // the DMA kernels address with 32-bit offsets: from the start of a gathered A,
    // from an expert's first weight row
    const uint64_t a_bytes = (uint64_t)a.a_rows * a.K * (a.a_dtype == MOE_ACT_MXFP8_E4M3 ? 1 : 2);
    if (a.a_gather && a_bytes >= (1ull << 32))
      return fail(MOE_ERR_SHAPE, "grouped GEMM: a gathered A of %llu bytes exceeds 4 GiB",
                  (unsigned long long)a_bytes);
    if ((uint64_t)a.N * (a.K / 2) >= (1ull << 32))
      return fail(MOE_ERR_SHAPE, "grouped GEMM: one expert's weights exceed 4 GiB");
  }
  if (!a.a_gather && a.a_rows < a.rows)
    return fail(MOE_ERR_SHAPE, "grouped GEMM: A has %d rows, fewer than rows %d", a.a_rows, a.rows);
  if (a.w_format != MOE_W_CANONICAL && a.w_format != MOE_W_TILED)
    return fail(MOE_ERR_INVALID_ARG, "grouped GEMM: bad w_format %d", a.w_format);
  if (a.w_format == MOE_W_TILED && (a.K % 512 || a.N % 256))
    return fail(MOE_ERR_SHAPE, "grouped GEMM: tiled weights need K %% 512 == 0 and N %% 256 == 0 (K %d, N %d)",
                a.K, a.N);
  return MOE_OK;
}

bool tile_shape_ok(int E, int N, int K) { return E >= 1 && N >= 256 && K >= 512 && N % 256 == 0 && K % 512 == 0; }

size_t tiled_bytes(int E, int N, int K, int which) {
  if (!tile_shape_ok(E, N, K) || (which != 0 && which != 1)) return 0;
  return (size_t)E * N * (which == 0 ? K / 2 : K / 32);
}

moe_status launch_tile(const uint8_t* src_p, const uint8_t* src_s, int E, int N, int K, int layout,
                       uint8_t* dst_p, uint8_t* dst_s, bool to_tiled, hipStream_t s) {
  const int grid = num_cus() * 8;
  if (to_tiled) {
    hipLaunchKernelGGL(tile_packed_kernel<true>, dim3(grid), dim3(256), 0, s, src_p, dst_p, E, N, K, layout);
    hipLaunchKernelGGL(tile_scales_kernel<true>, dim3(grid), dim3(256), 0, s, src_s, dst_s, E, N, K, layout);
  } else {
    hipLaunchKernelGGL(tile_packed_kernel<false>, dim3(grid), dim3(256), 0, s, src_p, dst_p, E, N, K, layout);
    hipLaunchKernelGGL(tile_scales_kernel<false>, dim3(grid), dim3(256), 0, s, src_s, dst_s, E, N, K, layout);
  }
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

moe_status launch_gemm(const moe_gemm_args& a, void* ws, hipStream_t s, int reserve, int max_rows) {
  if (a.rows == 0) return MOE_OK;
  const int cap = list_capacity(a.rows, a.E);
  Tile* lists = static_cast<Tile*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                               align_up(kClasses * (size_t)cap * sizeof(Tile), 256));
  // the three-stage DMA kernels need whole groups of four 128-element K stages;
  // other K use the register-staged kernels
  const bool dma = a.K % 512 == 0;
  const bool fp8 = a.a_dtype == MOE_ACT_MXFP8_E4M3;
  const int big_log2 = (dma && !fp8) ? 7 : 8;
  int32_t* unit_ctr = counts + 32;   // [class][xcd], inside the workspace's 256-byte count block
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a.expert_offsets, a.E, big_log2, lists, cap,
                     counts, unit_ctr);
  MXMOE_HIP(hipGetLastError());

  Params p{};
  p.unit_ctr = unit_ctr;
  p.a = static_cast<const uint8_t*>(a.a);
  p.a_scales = a.a_scales;
  p.a_gather = a.a_gather;
  p.a_gather_div = a.a_gather_div;
  if (a.a_gather) {
    // (validate_gemm keeps a gathered A below 4 GiB for the DMA kernels)
    const uint64_t row_bytes = (uint64_t)a.K * (a.a_dtype == MOE_ACT_MXFP8_E4M3 ? 1 : 2);
    p.a_bytes = (uint32_t)std::min<uint64_t>((uint64_t)a.a_rows * row_bytes, 0xffffffffull);
    p.as_bytes = (uint32_t)std::min<uint64_t>((uint64_t)a.a_rows * (a.K / 32), 0xffffffffull);
  }
  p.w = a.w_packed;
  p.w_scales = a.w_scales;
  p.offsets = a.expert_offsets;
  p.c = a.c;
  p.c_scales = a.c_scales;
  p.N = a.N;
  p.K = a.K;
  p.layout = a.epilogue;
  if (a.epilogue == MOE_EPI_NONE) {
    p.n_out = a.N;
    p.n_tiles = (a.N + kBN - 1) / kBN;
  } else {
    p.n_out = a.N / 2;
    p.n_tiles = (p.n_out + kBN / 2 - 1) / (kBN / 2);
  }
  const int path = !dma ? 0 : (a.w_format == MOE_W_TILED ? 2 : 1);
  // no expert holds more rows than the call (or than the caller's bound)
  const int mr = max_rows < 0 || max_rows > a.rows ? a.rows : max_rows;
  if (fp8) return dispatch_path<true>(path, p, a.epilogue, a.c_dtype, lists, cap, counts, s, reserve, mr);
  return dispatch_path<false>(path, p, a.epilogue, a.c_dtype, lists, cap, counts, s, reserve, mr);
}

}  // namespace mxmoe

#if MXMOE_PHASE_TIMERS
extern "C" {

// Phase timers (libmxmoe_phases.so only): zero them / copy them to host
// memory (unsigned long long [2048][4][12], layout as g_phase).  0 on success.
int mxmoe_phase_timers_reset() {
  static unsigned long long zero[mxmoe::kPhaseBlocks * mxmoe::kClasses * mxmoe::kPhaseSlots];
  return hipMemcpyToSymbol(HIP_SYMBOL(mxmoe::g_phase), zero, sizeof(zero)) == hipSuccess ? 0 : 1;
}
int mxmoe_phase_timers_read(void* host) {
  if (!host) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(mxmoe::g_phase), sizeof(mxmoe::g_phase)) == hipSuccess ? 0 : 1;
}

}  // extern "C"
#endif
