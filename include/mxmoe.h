/*
 * mxmoe.h -- C ABI of libmxmoe.so: a mixture-of-experts layer whose expert
 * weights are MXFP4, for AMD MI355X (gfx950).
 *
 * The layer, as the pages describe it:
 *   - top-k routing over E experts (256 experts / top-6 for the
 *     DeepSeek-V4-Flash shape: ktransformers issue #2172, "Environment";
 *     896 experts / top-16 for Kimi-K3: "Kimi-K3 SM120 FlashInfer MXFP4
 *     MoE", Phase-0 audit table);
 *   - dispatch of the routed tokens to the experts (issue #2172, "Impact");
 *   - expert FC1 (gate and up, twice FC2's inner width for a gated
 *     activation: Kimi-K3 page, on-machine evidence), the gated activation,
 *     expert FC2, with MXFP4 weights against bf16 or MXFP8 activations
 *     (Kimi-K3 page, goal; issue #2172 title);
 *   - the weighted top-k combine that ends a fused MoE (Kimi-K3 page, goal);
 *   - layerwise, double-buffered streaming of expert weights from host
 *     memory during prefill, instead of "load all experts, compute, hard
 *     sync" per layer (issue #2172, "Impact" and "Background / motivation").
 *
 * Number formats (OCP Microscaling Formats v1.0): an MXFP4 matrix [N][K] is
 * stored as packed FP4 E2M1 codes uint8 [N][K/2] (element 2j in the low
 * nibble, 2j+1 in the high nibble) plus E8M0 scales uint8 [N][K/32], one
 * per 32 consecutive elements along K.  MXFP8 activations are E4M3 codes
 * uint8 [rows][K] plus E8M0 scales uint8 [rows][K/32].  bf16 tensors are
 * passed as uint16 bit patterns.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device memory (or managed memory)
 *     on the current device; "host" pointers are host memory.  The caller
 *     owns every buffer, stream and event; the library never frees or
 *     keeps a pointer past the enqueued work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue: none waits for the device.
 *   - All argument checks run before anything is enqueued: a call that
 *     returns an error has enqueued nothing.  The detail of the last error
 *     on the calling thread is in moe_last_error_message().
 *   - Faults inside kernels surface at the caller's next synchronisation
 *     as HIP errors.
 *   - Only gfx950 devices are accepted (MOE_ERR_UNSUPPORTED_DEVICE
 *     otherwise); there is no fallback path.
 *   - The library reads no environment variables.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXMOE_ABI_VERSION 3

/* Every enum value is explicit and checked by the binding at load time:
 * a value that means one thing on one side of the boundary and another on
 * the other silently breaks gated activations (Kimi-K3 page, on-machine
 * evidence: the activation enum that disagreed between Python and C++). */
typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,       /* null pointer, bad enum value, negative size */
  MOE_ERR_SHAPE = 2,             /* sizes violate the layout rules stated per call */
  MOE_ERR_UNSUPPORTED_DEVICE = 3,/* current device is not gfx950 */
  MOE_ERR_NOT_PINNED = 4,        /* host weights are not page-locked */
  MOE_ERR_WORKSPACE = 5,         /* workspace missing or smaller than the size query */
  MOE_ERR_HIP = 6,               /* a HIP runtime call or launch failed */
  MOE_ERR_NOT_IMPLEMENTED = 7    /* a valid combination this build does not provide */
} moe_status;

typedef enum moe_act_dtype {     /* the A operand of a grouped GEMM */
  MOE_ACT_BF16 = 0,
  MOE_ACT_MXFP8_E4M3 = 1
} moe_act_dtype;

typedef enum moe_out_dtype {     /* the output of a grouped GEMM / intermediate */
  MOE_OUT_FP32 = 0,
  MOE_OUT_BF16 = 1,
  MOE_OUT_MXFP8_E4M3 = 2
} moe_out_dtype;

typedef enum moe_epilogue {
  MOE_EPI_NONE = 0,              /* C = A * W^T */
  MOE_EPI_SWIGLU_SPLIT = 1,      /* W rows [0,N/2) gate, [N/2,N) up; C[:, i] = silu(g_i) * u_i */
  MOE_EPI_SWIGLU_INTERLEAVED = 2 /* W row 2i gate, 2i+1 up; C[:, i] = silu(g_i) * u_i */
} moe_epilogue;

typedef enum moe_chain {         /* how stacked layers feed each other */
  MOE_CHAIN_RMS = 0,             /* x_{L+1}[t] = bf16(y_L[t] / rms(y_L[t])) */
  MOE_CHAIN_INDEPENDENT = 1      /* every layer reads x_0 */
} moe_chain;

typedef enum moe_weight_format { /* how a weight matrix and its scales sit in memory */
  MOE_W_CANONICAL = 0,           /* packed [E][N][K/2], scales [E][N][K/32] (row-major) */
  MOE_W_TILED = 1                /* the load-time tiling of moe_mxfp4_tile_weights */
} moe_weight_format;

typedef enum moe_expert_copy {   /* which experts the streamed prefill moves to HBM per layer */
  MOE_COPY_ALL = 0,              /* every expert of the layer (one copy-engine transfer) */
  MOE_COPY_ROUTED = 1,           /* only the experts the layer's routing hits (a copy kernel) */
  MOE_COPY_AUTO = 2              /* ROUTED when T <= routed_copy_max_tokens, else ALL */
} moe_expert_copy;

typedef enum moe_enum_kind {
  MOE_ENUM_STATUS = 0, MOE_ENUM_ACT = 1, MOE_ENUM_OUT = 2, MOE_ENUM_EPI = 3, MOE_ENUM_CHAIN = 4,
  MOE_ENUM_WFORMAT = 5, MOE_ENUM_COPY = 6
} moe_enum_kind;

/* ------------------------------------------------------------ queries -- */

int         moe_abi_version(void);
/* Static string for a status code; "unknown status" otherwise. */
const char* moe_status_string(int status);
/* Detail of the last failing call on this thread ("" if none).  Valid until
 * the next call on the same thread. */
const char* moe_last_error_message(void);
/* Name of enum value `value` of kind `kind` (e.g. "MOE_EPI_SWIGLU_SPLIT"),
 * or NULL if the value is not defined.  Lets a binding assert that its
 * mirror of every enum agrees with this header. */
const char* moe_enum_name(int kind, int value);
/* 1 if the current HIP device is a gfx950, 0 if not, -1 on a HIP error. */
int         moe_device_supported(void);

/* ------------------------------------------------------------ routing -- */

/* Top-k routing (the router of a top-k MoE: issue #2172 "Environment",
 * Kimi-K3 Phase-0 audit table).
 *   logits   device fp32 [T][E], row-major.
 *   topk_ids device int32 [T][k] out: expert ids, best first.  Order:
 *            logit descending, equal logits -> lower expert id first;
 *            -0.0 equals +0.0; NaN sorts after every number.
 *   topk_w   device fp32 [T][k] out: softmax over the E logits,
 *            renormalised over the k kept = exp(l_j - max) / sum_j'.
 * Sizes: T >= 0 (T == 0 enqueues nothing), 1 <= E <= 1024, 1 <= k <= min(E, 64).
 */
moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w, void* stream);

/* ------------------------------------------------------- permutation -- */

/* Bytes of device workspace moe_permute needs. */
size_t     moe_permute_workspace_size(int32_t T, int32_t E, int32_t k);

/* Stable counting sort of the T*k (token, slot) pairs by expert: the
 * dispatch of routed tokens to the experts (issue #2172, "Impact").
 *   topk_ids       device int32 [T][k], values in [0, E).
 *   expert_offsets device int32 [E+1] out: exclusive prefix sum of the
 *                  per-expert counts; expert_offsets[E] == T*k.
 *   perm_src       device int32 [T*k] out: permuted row r -> flat index
 *                  f = t*k + j; within an expert, rows are in increasing f.
 *   dest_row       device int32 [T*k] out: f -> permuted row (the inverse).
 *   workspace      device, >= moe_permute_workspace_size(T, E, k) bytes.
 * Sizes: T >= 0, 1 <= E <= 8192, 1 <= k <= E, T*k < 2^31.
 * Ids outside [0, E) are undefined behaviour (not checked on the device).
 */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                       int32_t* expert_offsets, int32_t* perm_src, int32_t* dest_row,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------- grouped MXFP4 GEMM -- */

typedef struct moe_gemm_args {
  const void*    a;              /* device: bf16 [a_rows][K] or E4M3 [a_rows][K] */
  const uint8_t* a_scales;       /* device E8M0 [a_rows][K/32] for MXFP8 A; NULL for bf16 */
  const int32_t* a_gather;       /* device int32 [rows] or NULL.  A row of permuted row r is
                                    a_gather[r] / a_gather_div (FC1 gathers token rows of x
                                    with perm_src and div = k); NULL: A row r */
  const uint8_t* w_packed;       /* device [E][N][K/2] packed E2M1 */
  const uint8_t* w_scales;       /* device [E][N][K/32] E8M0 */
  const int32_t* expert_offsets; /* device int32 [E+1] from moe_permute */
  void*          c;              /* device out [rows][N_out]: N_out = N/2 for SWIGLU, else N */
  uint8_t*       c_scales;       /* device out E8M0 [rows][N_out/32] for MXFP8 C; else NULL */
  int32_t        a_dtype;        /* moe_act_dtype */
  int32_t        a_gather_div;   /* >= 1 */
  int32_t        a_rows;         /* rows of A (T when gathering from x, else rows) */
  int32_t        rows;           /* permuted rows = expert_offsets[E] = T*k */
  int32_t        E, N, K;
  int32_t        epilogue;       /* moe_epilogue */
  int32_t        c_dtype;        /* moe_out_dtype (MXFP8 only with a SWIGLU epilogue) */
  int32_t        w_format;       /* moe_weight_format of w_packed / w_scales; MOE_W_TILED
                                    needs K % 512 == 0 and N % 256 == 0 and weights tiled
                                    with this call's epilogue */
} moe_gemm_args;

size_t     moe_grouped_gemm_workspace_size(const moe_gemm_args* args);

/* For every expert e with rows [off[e], off[e+1]):
 *   C[r][:] = epilogue( A[row(r)][:] . dequant(W[e])^T ),  dequant(W)[n][kk] =
 *   E2M1(code[n][kk]) * 2^(scale[n][kk/32] - 127), accumulated in fp32.
 * FC1 of the layer is this call with a SWIGLU epilogue (N = 2*I, K = H);
 * FC2 is this call with MOE_EPI_NONE (N = H, K = I).  bf16 A runs on bf16
 * MFMA with the weights expanded exactly to bf16; MXFP8 A runs on the
 * scaled FP8 x FP4 MFMA with both E8M0 scales applied inside it.
 * MXFP8 C (MOE_OUT_MXFP8_E4M3; SWIGLU epilogue and K % 512 == 0, else
 * MOE_ERR_NOT_IMPLEMENTED): each row's N_out values are cut into 32-element
 * blocks; a block with largest magnitude amax gets the E8M0 exponent X, the
 * smallest integer with amax * 2^-X <= 448 (so no element saturates;
 * clamped to [-127, 127]; amax == 0 gives X = -127), stored as X + 127 in
 * c_scales, and each element v becomes the E4M3 code nearest to v * 2^-X,
 * ties to even.  This is the intermediate of the MXFP8 x MXFP4 layer, which
 * FC2 then reads as MXFP8 A.
 * Shape rules (MOE_ERR_SHAPE): K % 32 == 0, N % 32 == 0, N % 64 == 0 for
 * SWIGLU, N_out % 32 == 0 for MXFP8 C, rows >= 0, 1 <= E; for K % 512 == 0
 * also a gathered A below 4 GiB and one expert's packed weights below 4 GiB.
 */
moe_status moe_mxfp4_grouped_gemm(const moe_gemm_args* args, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * grouped GEMM, with the same arguments, kernels and results as
 * moe_mxfp4_grouped_gemm, but its scratch (the planner's tile lists, tile
 * counts and unit counters) lives in a device array inside the library of
 * MXMOE_STATIC_SCRATCH_BYTES bytes, which each device the library runs on
 * holds until the process ends.  The call allocates and frees nothing.
 * Limit: moe_grouped_gemm_workspace_size(args) <= MXMOE_STATIC_SCRATCH_BYTES
 * (about rows / 32 + E <= 32 700; e.g. rows up to ~1 000 000 at E = 896),
 * MOE_ERR_WORKSPACE above it (nothing enqueued).  Every call on a device
 * shares that device's array: calls that overlap on one device (on different
 * streams, or from different threads) race and must not be issued; calls
 * ordered on one stream are safe.  The array keeps the last call's contents;
 * the planner rewrites every word the GEMM reads, so nothing needs clearing.
 * Errors as for moe_mxfp4_grouped_gemm. */
#define MXMOE_STATIC_SCRATCH_BYTES (1u << 20)
moe_status moe_mxfp4_grouped_gemm_static(const moe_gemm_args* args, void* stream);

/* ----------------------------------------------- load-time weight tiling -- */

/* Load-time repacking of one weight matrix into the order the grouped GEMM
 * streams it: the counterpart of the MXFP4 weight repack and E8M0 scale
 * swizzle that ktransformers issue #2172 (comments on the Marlin MoE path)
 * describes, where raw and repacked copies were both kept; here the caller
 * frees the canonical copy once the tiled one is made.  A 256-column slice of the
 * GEMM ("n-tile") over 128 K elements is one contiguous 16 KB block, already
 * in the slot order the kernels read from LDS, so every weight load is 1 KB
 * of consecutive bytes; an n-tile's E8M0 scales for 512 K elements are one
 * contiguous 4 KB block.  For a SWIGLU epilogue an n-tile holds 128 gate
 * rows and their 128 up rows, in groups of 32 gate then the 32 matching up
 * rows, so the tiling depends on the epilogue the matrix is used with (FC1:
 * its SWIGLU layout; FC2: MOE_EPI_NONE).
 *   w_packed, w_scales  device canonical [E][N][K/2], [E][N][K/32] (input)
 *   t_packed, t_scales  device out, moe_tiled_weight_bytes(E, N, K, 0 / 1)
 *                       bytes (the same byte counts as the canonical arrays)
 * Sizes: E >= 1, K % 512 == 0, N % 256 == 0 (MOE_ERR_SHAPE otherwise);
 * epilogue a moe_epilogue.  Input and output must not overlap.  Enqueued on
 * `stream`; nothing else is written.
 * moe_mxfp4_untile_weights is the exact inverse (tiled -> canonical), with
 * the same arguments in the other direction.
 * moe_tiled_weight_bytes returns 0 for sizes the tiling does not take.
 */
size_t     moe_tiled_weight_bytes(int32_t E, int32_t N, int32_t K, int32_t which);
moe_status moe_mxfp4_tile_weights(const uint8_t* w_packed, const uint8_t* w_scales, int32_t E, int32_t N,
                                  int32_t K, int32_t epilogue, uint8_t* t_packed, uint8_t* t_scales,
                                  void* stream);
moe_status moe_mxfp4_untile_weights(const uint8_t* t_packed, const uint8_t* t_scales, int32_t E, int32_t N,
                                    int32_t K, int32_t epilogue, uint8_t* w_packed, uint8_t* w_scales,
                                    void* stream);

/* ------------------------------------------------------------ combine -- */

/* Weighted top-k combine that ends the fused MoE (Kimi-K3 page, goal):
 *   out[t][h] = sum_{j = 0..k-1, ascending} topk_w[t][j] * y[dest_row[t*k+j]][h]
 * in fp32.  A gather-reduce: no atomics, run-to-run deterministic.
 *   y        device [T*k][H] in permuted row order, fp32 or bf16 (y_dtype).
 *   out      device fp32 [T][H].
 *   x_next   device bf16 [T][H] or NULL: if given, also writes
 *            bf16(out[t] / sqrt(mean_h out[t][h]^2)) (the stacked-layer
 *            rule MOE_CHAIN_RMS).
 * Sizes: T >= 0, k >= 1, H >= 1, H % 8 == 0.
 */
moe_status moe_combine(const void* y, int32_t y_dtype, const int32_t* dest_row,
                       const float* topk_w, int32_t T, int32_t k, int32_t H,
                       float* out, uint16_t* x_next, void* stream);

/* ------------------------------------------------ one resident layer -- */

typedef struct moe_layer_args {
  int32_t        T, H, I, E, k;
  int32_t        layout;         /* MOE_EPI_SWIGLU_SPLIT or MOE_EPI_SWIGLU_INTERLEAVED */
  int32_t        act_dtype;      /* moe_act_dtype of x */
  int32_t        inter_dtype;    /* moe_out_dtype of the SwiGLU output fed to FC2:
                                    MOE_OUT_BF16 or MOE_OUT_MXFP8_E4M3 */
  const float*   logits;         /* device fp32 [T][E] */
  const void*    x;              /* device bf16 [T][H] or E4M3 [T][H] */
  const uint8_t* x_scales;       /* device E8M0 [T][H/32] (MXFP8 x only) */
  const uint8_t* w1_packed;      /* device [E][2I][H/2] */
  const uint8_t* w1_scales;      /* device [E][2I][H/32] */
  const uint8_t* w2_packed;      /* device [E][H][I/2] */
  const uint8_t* w2_scales;      /* device [E][H][I/32] */
  float*         out;            /* device fp32 [T][H] */
  uint16_t*      x_next;         /* device bf16 [T][H] or NULL (see moe_combine) */
  void*          workspace;      /* device, >= moe_layer_workspace_size() */
  size_t         workspace_bytes;
  int32_t        w_format;       /* moe_weight_format of both weight matrices (tiled: W1
                                    with `layout`, W2 with MOE_EPI_NONE) */
} moe_layer_args;

/* Bytes of workspace for a layer of these sizes (routing arrays, the
 * intermediate and FC2's output included). */
size_t     moe_layer_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                    int32_t inter_dtype);

/* Byte offsets, inside the layer workspace, of the routing arrays the layer
 * writes (for inspection after the call): which = 0 topk_ids, 1 topk_w,
 * 2 expert_offsets, 3 perm_src, 4 dest_row.  (size_t)-1 for a bad `which`. */
size_t     moe_layer_workspace_offset(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                      int32_t inter_dtype, int32_t which);

/* route -> permute -> FC1 + SwiGLU -> FC2 -> combine, all on `stream`. */
moe_status moe_layer_forward(const moe_layer_args* args, void* stream);

/* ------------------------------------------------ captured layer ------ */

/* Graph capture and replay of one resident layer ("Kimi-K3 SM120 FlashInfer
 * MXFP4 MoE" page, Phase-1 gates, item 5: token counts 1/2/8/32 under graph
 * capture/replay).
 *
 * moe_layer_graph_create validates *args exactly as moe_layer_forward does,
 * captures one moe_layer_forward(args) on `stream` into a HIP graph and
 * instantiates it.  Nothing runs during the capture.  The graph keeps every
 * pointer of *args (not the struct itself): a replay reads the inputs'
 * contents at replay time and writes the same outputs and workspace, so
 * replays on one handle must not overlap each other or a moe_layer_forward
 * on the same workspace.  T, the weights and the workspace are fixed per
 * handle.  `stream` must be a created stream (capture on the null stream
 * is MOE_ERR_INVALID_ARG) with no other capture in progress; it is left in
 * normal (non-capturing) mode on every return.  On failure *graph is NULL
 * and the status is forward's (or MOE_ERR_HIP for a capture/instantiate
 * failure).  The handle is host memory owned by the caller until
 * moe_layer_graph_destroy.
 *
 * moe_layer_graph_launch enqueues one replay on `stream` (any stream of the
 * device the graph was captured on; MOE_ERR_INVALID_ARG on another device).
 * Output ordering is that of a kernel launch on `stream`.
 *
 * moe_layer_graph_destroy frees the handle (NULL is accepted); the caller
 * first makes sure no replay is still running.
 */
typedef struct moe_layer_graph moe_layer_graph;
moe_status moe_layer_graph_create(const moe_layer_args* args, void* stream, moe_layer_graph** graph);
moe_status moe_layer_graph_launch(moe_layer_graph* graph, void* stream);
moe_status moe_layer_graph_destroy(moe_layer_graph* graph);

/* ------------------------------------------------ streamed prefill ---- */

typedef struct moe_streamed_args {
  int32_t        num_layers, T, H, I, E, k;
  int32_t        layout;         /* MOE_EPI_SWIGLU_SPLIT or _INTERLEAVED */
  int32_t        chain;          /* moe_chain */
  int32_t        depth;          /* 2: double-buffered (copy of L+1 overlaps compute of L);
                                    1: serialized (copy, compute, copy, ...) for comparison */
  int32_t        num_blobs;      /* distinct host blobs; layer L uses blob L % num_blobs */
  const void* const* host_blobs; /* host array of num_blobs page-locked host pointers; each
                                    blob = W1p | S1 | W2p | S2, each section starting at a
                                    multiple of 256 bytes (moe_blob_section_offset) */
  size_t         blob_bytes;     /* >= moe_blob_bytes(H, I, E) */
  void*          device_slot[2]; /* device, each >= blob_bytes (slot[1] unused at depth 1) */
  const float*   logits;         /* device fp32 [num_layers][T][E] */
  const uint16_t* x;             /* device bf16 [T][H]: the first layer's input */
  float*         out;            /* device fp32 [T][H]: the last layer's output */
  uint16_t*      layer_inputs;   /* device bf16 [num_layers][T][H] or NULL: every layer's
                                    input, recorded for per-layer checks */
  void*          events;         /* host array of num_layers*4 hipEvent_t or NULL: recorded at
                                    copy start, copy end (copy stream), compute start, compute
                                    end (compute stream) of every layer */
  void*          workspace;      /* device, >= moe_streamed_workspace_size() */
  size_t         workspace_bytes;
  int32_t        w_format;       /* moe_weight_format of the blobs' W1/S1 and W2/S2 sections */
  int32_t        expert_copy;    /* moe_expert_copy */
  int32_t        routed_copy_max_tokens; /* MOE_COPY_AUTO: the largest T that copies routed
                                    experts only (the token threshold below which a
                                    layer's batch leaves most experts unused) */
} moe_streamed_args;

/* Bytes of one layer's weight blob, and the byte offset of its sections:
 * which = 0 W1p, 1 S1, 2 W2p, 3 S2. */
size_t     moe_blob_bytes(int32_t H, int32_t I, int32_t E);
size_t     moe_blob_section_offset(int32_t H, int32_t I, int32_t E, int32_t which);
size_t     moe_streamed_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/* Layerwise streamed prefill (issue #2172, "Background / motivation": the
 * double-buffered layerwise pipeline that replaces the serialized
 * per-layer H2D chain).  For L = 0..num_layers-1: the copy stream fills
 * slot (L % 2) with blob (L % num_blobs) once the compute of layer L-2
 * (the slot's previous user) is done; the compute stream waits for that
 * copy and runs the layer.  The copy stream first waits for the compute
 * stream's earlier work.  Nothing waits on the host; on return both
 * streams hold the whole pass and `out` is ordered on `compute`.
 * MOE_ERR_NOT_PINNED if a blob is not page-locked host memory.  At depth 2
 * the two streams must differ (MOE_ERR_INVALID_ARG otherwise: on one
 * stream every copy would wait for the previous layer's compute).
 *
 * Routed expert copy (MOE_COPY_ROUTED, or MOE_COPY_AUTO with
 * T <= routed_copy_max_tokens): the router logits of every layer are inputs
 * of the call, so layer L's routing is known before layer L-1 ends.  The
 * copy stream then routes and permutes layer L itself (into its own
 * double-buffered routing arrays) and moves only the experts with at least
 * one routed row, with a kernel that reads the blob through its
 * device-mapped address (a blob that has none is MOE_ERR_NOT_PINNED); the
 * compute stream runs FC1, FC2 and the combine on that routing.  The
 * experts the layer does not hit keep whatever the slot held before: no
 * kernel reads them.  The GEMMs then leave one CU per XCD free for the copy
 * kernel.  Outputs are bitwise those of MOE_COPY_ALL.  Blob and slot
 * addresses must be 16-byte aligned (MOE_ERR_INVALID_ARG otherwise).
 */
moe_status moe_layer_prefill_streamed(const moe_streamed_args* args, void* compute_stream,
                                      void* copy_stream);

#ifdef __cplusplus
}
#endif
#endif /* MXMOE_H */
