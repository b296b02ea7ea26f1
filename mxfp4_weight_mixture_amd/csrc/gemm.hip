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
// into 256-row tiles plus one remainder tile, and files every tile under
// one of four row-tile sizes (32, 64, 128, 256) so that an expert with a
// handful of rows (the decode shapes, the tail of a skewed routing) does
// not pay for 256 rows of matrix-core work.  One persistent launch per tile
// size walks its list; a (tile, n-tile) unit is one 256-column slice of one
// row tile.  Units are dealt to the 8 XCDs in contiguous ranges, n-tile
// fastest, so that the blocks sharing an XCD's L2 work on the same rows.
//
// Block: 256 threads = 4 wave64s.  Per K stage (128 bytes of each A row:
// 128 FP8 or 64 bf16 elements) the A tile, the B tile and their scales go
// global -> registers -> LDS (double-buffered, one barrier per stage); the
// global loads for stage s+1 are in flight while stage s is multiplied.
// LDS rows are padded by 16 bytes so that the 16-byte fragment reads of 8
// consecutive rows land on distinct banks.
//
// MFMA operand layout used (32x32 tiles, measured on gfx950 with one-hot
// operands): lane l supplies row/column (l % 32).  For the scaled
// 32x32x64 MFMA, an FP4 B lane in half g = l/32 holds K [32g, 32g+32) (one
// whole MX block), an FP8 A lane in half g holds K [16g, 16g+16) followed by
// K [32+16g, 32+16g+16), and the E8M0 scale supplied by a lane in half g
// applies to K block g of its row/column.  For the bf16 32x32x16 MFMA a
// lane in half g holds K [8g, 8g+8).  Accumulator j of lane l is
// C[8*(j/4) + 4*(l/32) + j%4][l % 32].
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
  const Tile* tiles;
  const int32_t* tile_count;
  int a_gather_div;
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

// Row of W (within one expert) that feeds tile column j of n-tile nt.
template <int WN>
__device__ inline int w_row_of(int layout, int nt, int j, int N, int n_out) {
  if (layout == 0) {
    const int n = nt * kBN + j;
    return n < N ? n : N - 1;
  }
  // SwiGLU: each wave's WN columns are WN/2 gate rows then the WN/2 matching up rows
  const int hp = WN / 2;
  const int i = nt * (kBN / 2) + (j / WN) * hp + (j % WN) % hp;
  const bool up = (j % WN) >= hp;
  if (i >= n_out) return 0;
  if (layout == 1) return up ? n_out + i : i;
  return up ? 2 * i + 1 : 2 * i;
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

template <int BM, bool FP8>
struct Cfg2 {
  static constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
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
  static constexpr int A_I = BM * RA / 4096;        // A DMA instructions per wave per stage
  static constexpr int B_I = kBN * RB / 4096;       // B DMA instructions per wave per stage (4)
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

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, bool FP8, int EPI, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_dma_kernel(Params p) {
  using C = Cfg2<BM, FP8>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / C::WAVES_N) * C::WM;
  const int wn0 = (wave % C::WAVES_N) * C::WN;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  // fragment rows / lines start at multiples of 16, so the swizzles depend on the lane only
  const int xa = a_swz<FP8>(l32 & 15);
  const int xb = b_swz((l32 >> 1) & 7);

  const int count = *p.tile_count;
  const int units = count * p.n_tiles;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int u_end = min(units, (xcd + 1) * per_xcd);

  const int K = p.K;
  const int a_row_bytes = FP8 ? K : 2 * K;
  const int kb = K / 32;
  const int nst = K / C::KS;

  for (int u = xcd * per_xcd + slot; u < u_end; u += slots) {
    // units in groups of up to 4 row tiles x all n-tiles, row tile fastest, so
    // that concurrent blocks of one XCD share both their A rows and their B tiles
    constexpr int GM = 4;
    const int grp = u / (GM * p.n_tiles);
    const int first = grp * GM;
    const int gsize = min(GM, count - first);
    const int in = u - grp * GM * p.n_tiles;
    const int ti = first + in % gsize;
    const int nt = in / gsize;
    const Tile tile = p.tiles[ti];
    const int e = tile.expert;
    const int row0 = tile.row0;
    const int mrows = min(BM, p.offsets[e + 1] - row0);
    const size_t w_expert = (size_t)e * p.N;

    // ---- per-lane DMA sources (stage 0; stage s adds s * bytes-per-stage) ----
    const uint8_t* a_src[C::A_I];
#pragma unroll
    for (int i = 0; i < C::A_I; ++i) {
      const int r = (wave * C::A_I + i) * C::A_ROWS_PER_I + lane / C::SA;
      const int chunk = (lane % C::SA) ^ a_swz<FP8>(r);
      const int grow = row0 + min(r, mrows - 1);
      const int arow = p.a_gather ? p.a_gather[grow] / p.a_gather_div : grow;
      a_src[i] = p.a + (size_t)arow * a_row_bytes + chunk * 16;
    }
    const uint8_t* b_src[C::B_I];
#pragma unroll
    for (int i = 0; i < C::B_I; ++i) {
      const int line = (wave * C::B_I + i) * 8 + lane / 8;
      const int uu = (lane & 7) ^ b_swz(line);
      const int j = line * 2 + (uu >> 2);
      const int wr = w_row_of<C::WN>(p.layout, nt, j, p.N, p.n_out);
      b_src[i] = p.w + (w_expert + wr) * (size_t)(K / 2) + (uu & 3) * 16;
    }
    const int srow = wave * 64 + lane;   // scale row this lane loads (A: if < BM)
    const uint8_t* as_src = nullptr;
    if (FP8 && srow < BM) {
      const int grow = row0 + min(srow, mrows - 1);
      const int arow = p.a_gather ? p.a_gather[grow] / p.a_gather_div : grow;
      as_src = p.a_scales + (size_t)arow * kb;
    }
    const uint8_t* bs_src =
        p.w_scales + (w_expert + w_row_of<C::WN>(p.layout, nt, srow, p.N, p.n_out)) * (size_t)kb;
    uint8_t* const sg = lds + C::NST * C::LDS_STAGE;   // two scale groups

    auto issue = [&](int s) {
      uint8_t* base = lds + (s % C::NST) * C::LDS_STAGE;
#pragma unroll
      for (int i = 0; i < C::A_I; ++i)
        lds_dma16(a_src[i] + (size_t)s * C::RA, base + (wave * C::A_I + i) * 1024);
#pragma unroll
      for (int i = 0; i < C::B_I; ++i)
        lds_dma16(b_src[i] + (size_t)s * C::RB, base + C::LDS_A + (wave * C::B_I + i) * 1024);
    };
    // scale group j (stages 4j..4j+3): 16 bytes of every A and B row
    auto issue_scales = [&](int j) {
      uint8_t* base = sg + (j & 1) * C::LDS_SG;
      if (FP8 && wave * 64 < BM) {
        if (as_src) lds_dma16(as_src + 16 * j, base + wave * 1024);
      }
      lds_dma16(bs_src + 16 * j, base + C::SG_A + wave * 1024);
    };

    v16f acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    issue_scales(0);
    issue(0);
    if (nst > 1) issue(1);

    for (int s = 0; s < nst; ++s) {
      // loads issued after stage s's: stage s+1's (and possibly a scale group); waiting
      // for fewer outstanding than that is conservative
      if (s + 1 < nst) wait_vm<C::LOADS>();
      else wait_vm<0>();
      stage_barrier();
      if (s + 2 < nst) {
        issue(s + 2);
        if (((s + 2) & 3) == 0) issue_scales((s + 2) >> 2);
      }
      const uint8_t* base = lds + (s % C::NST) * C::LDS_STAGE;
      const uint8_t* la = base;
      const uint8_t* lb = base + C::LDS_A;
      const uint8_t* lsg = sg + ((s >> 2) & 1) * C::LDS_SG + (s & 3) * 4;
      const uint8_t* lsa = lsg;
      const uint8_t* lsb = lsg + C::SG_A;
      // four scale bytes (this stage's blocks) per fragment row / column
      uint32_t bsw[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        bsw[fn] = *reinterpret_cast<const uint32_t*>(lsb + (wn0 + fn * 32 + l32) * 16);
      if constexpr (FP8) {
        uint32_t asw[C::FM];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
          asw[fm] = *reinterpret_cast<const uint32_t*>(lsa + (wm0 + fm * 32 + l32) * 16);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          v8i af[C::FM];
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm) {
            const uint8_t* row = la + (wm0 + fm * 32 + l32) * C::RA;
            // K [kk*64 + 16g, +16) and [kk*64 + 32 + 16g, +16): chunks 4kk+g and 4kk+2+g
            const v4i lo = *reinterpret_cast<const v4i*>(row + (((4 * kk + g) ^ xa) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(row + (((4 * kk + 2 + g) ^ xa) << 4));
            af[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) {
            const int n = wn0 + fn * 32 + l32;
            const int uu = ((n & 1) * 4 + 2 * kk + g) ^ xb;
            const v4i bq = *reinterpret_cast<const v4i*>(lb + (n >> 1) * 128 + (uu << 4));
            const v8i bf = v8i{bq[0], bq[1], bq[2], bq[3], 0, 0, 0, 0};
            const int bsc = (bsw[fn] >> (8 * (2 * kk + g))) & 0xff;
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
              const int asc = (asw[fm] >> (8 * (2 * kk + g))) & 0xff;
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af[fm], bf, acc[fm][fn], 0 /*A: fp8 e4m3*/, 4 /*B: fp4 e2m1*/, 0, asc, 0, bsc);
            }
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // this lane's 32 weights of block 2h+g, expanded to bf16
          v8bf bw[C::FN][4];
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) {
            const int n = wn0 + fn * 32 + l32;
            const int uu = ((n & 1) * 4 + 2 * h + g) ^ xb;
            const v4i bq = *reinterpret_cast<const v4i*>(lb + (n >> 1) * 128 + (uu << 4));
            const float sc = e8m0_to_f32((bsw[fn] >> (8 * (2 * h + g))) & 0xff);
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
              const uint8_t* row = la + (wm0 + fm * 32 + l32) * C::RA;
              // bytes 128h + 64g + 16*s4 of the 256-byte stage row: slot 8h + 4g + s4
              af[fm] = *reinterpret_cast<const v8bf*>(row + (((8 * h + 4 * g + s4) ^ xa) << 4));
            }
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
              for (int fm = 0; fm < C::FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bw[fn][s4], acc[fm][fn],
                                                                      0, 0, 0);
          }
        }
      }
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
            const float a = __fdividef(gv, 1.0f + __expf(-gv)) * uv;
            if (r < mrows && i < p.n_out) {
              const size_t o = (size_t)(row0 + r) * p.n_out + i;
              if (OUT == MOE_OUT_FP32) static_cast<float*>(p.c)[o] = a;
              else static_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(a);
            }
          }
        }
    }
    // every wave is done reading the stage buffers before the next unit refills them
    stage_barrier();
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
                                                    int32_t* __restrict__ counts) {
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
int persistent_grid(KernelT kernel) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = num_cus() * per_cu;
  return (grid + kXcds - 1) / kXcds * kXcds;
}

template <int BM, bool FP8, int EPI, int OUT, bool DMA>
moe_status launch_class(const Params& p, hipStream_t s) {
  static int grid = 0;  // per instantiation; one device type (gfx950)
  if constexpr (DMA) {
    if (grid == 0) grid = persistent_grid(gemm_dma_kernel<BM, FP8, EPI, OUT>);
    hipLaunchKernelGGL((gemm_dma_kernel<BM, FP8, EPI, OUT>), dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    if (grid == 0) grid = persistent_grid(gemm_kernel<BM, FP8, EPI, OUT>);
    hipLaunchKernelGGL((gemm_kernel<BM, FP8, EPI, OUT>), dim3(grid), dim3(kThreads), 0, s, p);
  }
  MXMOE_HIP(hipGetLastError());
  return MOE_OK;
}

template <bool FP8, int EPI, int OUT, bool DMA>
moe_status launch_all(Params p, const Tile* lists, int cap, const int32_t* counts, hipStream_t s) {
  p.tiles = lists + 0 * cap; p.tile_count = counts + 0;
  MXMOE_TRY((launch_class<32, FP8, EPI, OUT, DMA>(p, s)));
  p.tiles = lists + 1 * cap; p.tile_count = counts + 1;
  MXMOE_TRY((launch_class<64, FP8, EPI, OUT, DMA>(p, s)));
  p.tiles = lists + 2 * cap; p.tile_count = counts + 2;
  MXMOE_TRY((launch_class<128, FP8, EPI, OUT, DMA>(p, s)));
  // the bf16 DMA kernel's full tile is 128 rows, so its class-3 list is empty
  if constexpr (!(DMA && !FP8)) {
    p.tiles = lists + 3 * cap; p.tile_count = counts + 3;
    MXMOE_TRY((launch_class<256, FP8, EPI, OUT, DMA>(p, s)));
  }
  return MOE_OK;
}

template <bool FP8, int EPI, bool DMA>
moe_status dispatch_out(const Params& p, int c_dtype, const Tile* lists, int cap,
                        const int32_t* counts, hipStream_t s) {
  if (c_dtype == MOE_OUT_FP32) return launch_all<FP8, EPI, MOE_OUT_FP32, DMA>(p, lists, cap, counts, s);
  if (c_dtype == MOE_OUT_BF16) return launch_all<FP8, EPI, MOE_OUT_BF16, DMA>(p, lists, cap, counts, s);
  return fail(MOE_ERR_NOT_IMPLEMENTED, "grouped GEMM: MXFP8 output is not provided by this build");
}

template <bool FP8, bool DMA>
moe_status dispatch_epi(const Params& p, int epi, int c_dtype, const Tile* lists, int cap,
                        const int32_t* counts, hipStream_t s) {
  if (epi == MOE_EPI_NONE) return dispatch_out<FP8, 0, DMA>(p, c_dtype, lists, cap, counts, s);
  return dispatch_out<FP8, 1, DMA>(p, c_dtype, lists, cap, counts, s);
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
  if (a.c_dtype == MOE_OUT_MXFP8_E4M3)
    return fail(MOE_ERR_NOT_IMPLEMENTED, "grouped GEMM: MXFP8 output is not provided by this build");
  if (!a.a_gather && a.a_rows < a.rows)
    return fail(MOE_ERR_SHAPE, "grouped GEMM: A has %d rows, fewer than rows %d", a.a_rows, a.rows);
  return MOE_OK;
}

moe_status launch_gemm(const moe_gemm_args& a, void* ws, hipStream_t s) {
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
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a.expert_offsets, a.E, big_log2, lists, cap,
                     counts);
  MXMOE_HIP(hipGetLastError());

  Params p{};
  p.a = static_cast<const uint8_t*>(a.a);
  p.a_scales = a.a_scales;
  p.a_gather = a.a_gather;
  p.a_gather_div = a.a_gather_div;
  p.w = a.w_packed;
  p.w_scales = a.w_scales;
  p.offsets = a.expert_offsets;
  p.c = a.c;
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
  if (fp8)
    return dma ? dispatch_epi<true, true>(p, a.epilogue, a.c_dtype, lists, cap, counts, s)
               : dispatch_epi<true, false>(p, a.epilogue, a.c_dtype, lists, cap, counts, s);
  return dma ? dispatch_epi<false, true>(p, a.epilogue, a.c_dtype, lists, cap, counts, s)
             : dispatch_epi<false, false>(p, a.epilogue, a.c_dtype, lists, cap, counts, s);
}

}  // namespace mxmoe
