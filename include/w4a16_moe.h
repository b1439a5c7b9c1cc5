/*
 * w4a16_moe.h -- C ABI of the MI355X (gfx950) local W4A16 mixture-of-experts
 * forward pass.
 *
 * Sources (web pages, cited by tag and section):
 *   [P1] lmdeploy PR #4947, "feat(pytorch): add CuTeDSL W4A16 MoE backend"
 *   [P2] flashinfer PR #5186, "perf: reduce split W4A16 routing and output
 *        overhead"
 *   [P3] TensorRT-LLM PR #18313, "Add W4A16 per-channel weight-only support
 *        for Cutlass fused MoE"
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Tensors are
 *     row-major and contiguous.  Activations, packed weights, outputs and the
 *     workspace must be 16-byte aligned, scales 4-byte aligned.
 *   - 16-bit floating-point tensors (x, scales, out) all share desc->dtype.
 *   - Nothing is allocated per call and nothing synchronizes: work is enqueued
 *     on `stream` (0 = the null stream) and the call returns.  No device value
 *     is read back, so a call can be captured in a HIP graph.
 *   - Argument checking happens on the host before anything is enqueued.  A
 *     rejected call enqueues nothing and returns a status; the thread-local
 *     w4a16_last_error_message() then names the offending tensor or field.
 *     Launch failures return W4A16_ERR_HIP.  Faults inside kernels surface at
 *     the caller's next synchronization, like any HIP error.
 *   - A route whose expert id is outside [expert_offset, expert_offset + E) is
 *     an invalid route, not an error: it contributes nothing ([P1]
 *     Modification, "invalid routes and masked expert counts").
 *   - Calls on distinct workspaces are independent; two calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef W4A16_MOE_H
#define W4A16_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* w4a16_stream_t; /* a hipStream_t */

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1,          /* malformed descriptor or pointer    */
  W4A16_ERR_UNSUPPORTED = 2,          /* well-formed but not implemented    */
  W4A16_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the required */
  W4A16_ERR_HIP = 4                   /* a HIP launch call failed           */
} w4a16_status_t;

typedef enum { W4A16_DT_BF16 = 0, W4A16_DT_FP16 = 1 } w4a16_dtype_t;

/* Expert activation: gated SiLU(gate) * up over a fused gate/up weight whose
 * rows [0, I) are gate and [I, 2I) are up ([P1] Benchmark, timed steps), or
 * the non-gated ReLU^2 = max(h, 0)^2 over a single up weight ([P3]
 * Validation). */
typedef enum { W4A16_ACT_SILU_GATED = 0, W4A16_ACT_RELU2 = 1 } w4a16_act_t;

/* Weight quantization layout ([P3] Checkpoint format for the packing rule:
 * two INT4 per byte, even logical index in the low nibble, symmetric
 * two's-complement values, scale = absmax / 7).
 *   GROUP_K      one 16-bit scale per group_size (= 32) consecutive values of
 *                the reduction dim, packed along the reduction dim
 *                ([P1] BC-breaking, "INT4 group-size 32").
 *   PER_CHANNEL  one 16-bit scale per output channel, packed along the output
 *                dim ([P3] Description and Checkpoint format).
 *   FP4_GROUP_K  FP4 weights: E2M1 codes (OCP microscaling element format: sign,
 *                2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5,
 *                1, 1.5, 2, 3, 4, 6) in the GROUP_K layout, two per byte along K,
 *                one 16-bit scale per 32 values; W = e2m1 * scale, exact.  An
 *                MXFP4 checkpoint's E8M0 scales 2^(e-127) convert exactly with
 *                w4a16_e8m0_to_scales.  The 4-bit floating-point weights of
 *                [P2] Final performance (NVFP4, BF16 activations) in the block
 *                format gfx950 supports natively. */
typedef enum { W4A16_Q_GROUP_K = 0, W4A16_Q_PER_CHANNEL = 1, W4A16_Q_FP4_GROUP_K = 2 } w4a16_qlayout_t;

/* Problem descriptor (host memory, read during the call only).
 *   Logical weight shapes, with N1 = 2*I for SILU_GATED and N1 = I for RELU2:
 *     w13 [E][N1][H]   (gate/up, or w1)       w2 [E][H][I]   (down)
 *   Packed storage:
 *     GROUP_K and FP4_GROUP_K:
 *                   w13_packed u8 [E][N1][H/2],   w13_scales [E][N1][H/32]
 *                   w2_packed  u8 [E][H][I/2],    w2_scales  [E][H][I/32]
 *     PER_CHANNEL:  w13_packed u8 [E][N1/2][H],   w13_scales [E][N1]
 *                   w2_packed  u8 [E][H/2][I],    w2_scales  [E][H]
 *   Supported: H and I multiples of 64, 1 <= E <= 1024, 1 <= top_k <= 32,
 *   group_size 32 for GROUP_K, x below 2^31 bytes, one expert's w13 below
 *   2^30 bytes.
 *   force_* fields select a variant for testing; 0 means "choose from the
 *   route count".  Every variant computes the same function. */
typedef struct {
  int32_t num_tokens;         /* T >= 0; T = 0 enqueues nothing                   */
  int32_t hidden;             /* H                                                */
  int32_t intermediate;       /* I                                                */
  int32_t num_local_experts;  /* E                                                */
  int32_t expert_offset;      /* global id of local expert 0                      */
  int32_t top_k;              /* K                                                */
  int32_t group_size;         /* 32 for GROUP_K, ignored for PER_CHANNEL          */
  int32_t dtype;              /* w4a16_dtype_t                                    */
  int32_t act;                /* w4a16_act_t                                      */
  int32_t qlayout;            /* w4a16_qlayout_t                                  */
  int32_t force_path;         /* 0, 1 = grouped (route preparation, expert tiles,
                                 down GEMM, combine kernel), 2 = small batch (no
                                 route preparation; needs T*K <= 128)            */
  int32_t force_block_m;      /* grouped path: 0 or 64 (rows per expert tile;
                                 tiles are always 64 rows, empty 16-row subtiles
                                 skipped)                                        */
  int32_t force_splitk;       /* grouped path with 64-row tiles: 0 = choose from
                                 the expected routes per expert, 1 = split-K
                                 gate/up (partials + activation kernel), 2 = the
                                 streaming gate/up kernel                        */
  int32_t num_global_experts; /* experts the routes are drawn over (a local share
                                 of E of them); only the variant choice uses it
                                 (expected valid routes per local expert): ids
                                 are not checked against it, any id outside
                                 the local range is an invalid route.
                                 0 = E; otherwise >= E                           */
  int32_t fp16_route;         /* 0 (default): every product is formed with
                                 exact per-group scaling, for every finite
                                 input.  1: opt in to the fp16 route (bf16
                                 activations, bf16 group scales, 16 or more
                                 expected routes per expert): activations are
                                 staged as fp16, so an activation below 2^-14
                                 in magnitude is rounded to a multiple of
                                 2^-24 (an absolute error of at most 2^-25);
                                 a row made only of such values keeps fewer
                                 bits.  Activations of 2^16 or more and scales
                                 outside 2^-17..2720 are detected and those
                                 tiles recomputed per group                      */
  int32_t fused_finalize;     /* grouped path, the two finalize modes of [P2]
                                 Description: 0 (default) non-fused, the 16-bit
                                 expert outputs then a combine launch of its
                                 own; 1 fused, the combine inside the down GEMM
                                 launch (the workgroup whose arrival completes a
                                 token's routes for a column chunk combines it;
                                 not with the opted-in fp16 down route).  Same
                                 bits either way; the fused mode is slower on
                                 MI355X (one L2 write-back per workgroup).      */
  int32_t force_tile_order;   /* grouped path: 0 = choose from the expected
                                 routes per expert, 1 = tiles in route order, 2 =
                                 the tile launches (streaming gate/up, down)
                                 take tiles by descending count of non-empty
                                 16-row subtiles, written by route preparation.
                                 Same bits either way.                           */
} w4a16_moe_desc_t;

/* Variant the library runs for a descriptor (for tests and reports). */
typedef struct {
  int32_t path;               /* 1 grouped, 2 small batch                        */
  int32_t block_m;            /* grouped path: rows per expert tile              */
  int32_t k_slice;            /* gate/up reduction slice per wave (8 waves split
                                 the reduction when tiles have few rows)         */
  int32_t splitk_chunks;      /* split-K gate/up: reduction chunks (0 = off)     */
  int64_t max_positions;      /* capacity of the padded route list               */
  int64_t max_tiles;          /* capacity of the expert tile list                */
  size_t workspace_bytes;     /* bytes w4a16_moe_forward needs                   */
  int32_t fp16_route;         /* bit 0: the streaming gate/up tiles take the
                                 exact fp16 route (bf16 activations, bf16 group
                                 scales, enough routes per expert); bit 1: so
                                 does the down GEMM                              */
  int32_t rerun_flags_up;     /* int32 flags the gate/up fp16-route launch
                                 writes (one per workgroup, 1 = its tile met an
                                 activation of magnitude 2^16 or more, or a
                                 group scale outside 2^-17..2720, and was rerun
                                 per group); 0 if none                           */
  int32_t rerun_flags_down;   /* likewise for the down GEMM                      */
  int32_t fused_combine;      /* 1: the combine runs inside the down launch
                                 (fused finalize)                                */
  size_t rerun_flags_offset;  /* workspace byte offset of the flags: the gate/up
                                 launch's rerun_flags_up flags, then the down
                                 launch's rerun_flags_down (0 if neither launch
                                 exists)                                         */
  int32_t tile_order;         /* 1: the tile launches take tiles biggest first   */
  int32_t act_in_down;        /* 1: split-K gate/up, and the down launch forms
                                 the activations from its partials (no
                                 activation launch)                              */
} w4a16_moe_plan_t;

/* Bytes of device workspace w4a16_moe_forward needs for this descriptor
 * (depends on num_tokens: token counts stay dynamic while layouts are fixed,
 * [P2] Description, "Contract"; the caller owns the scratch the non-fused
 * finalization stores its 16-bit expert outputs in, same section).  Errors as
 * for the forward's checks; *bytes is written only on W4A16_OK. */
w4a16_status_t w4a16_moe_workspace_size(const w4a16_moe_desc_t* desc, size_t* bytes);

/* The variant the forward will run for this descriptor. */
w4a16_status_t w4a16_moe_get_plan(const w4a16_moe_desc_t* desc, w4a16_moe_plan_t* plan);

/* The local W4A16 fused-MoE forward ([P1] Benchmark: route preparation,
 * gate/up GEMM, SiLU, down GEMM and weighted reduction; [P2] Description,
 * "Contract": FP32 combine in fixed top-k order before one 16-bit cast).
 *   x             [T][H]  16-bit activations
 *   w13_*, w2_*   packed INT4 weights and 16-bit scales, layouts above
 *   topk_ids      [T][K]  int32 global expert ids (out-of-range -> invalid)
 *   topk_weights  [T][K]  fp32 routing weights, applied as given
 *   out           [T][H]  16-bit; out[t] = cast16(sum over k ascending of
 *                 topk_weights[t][k] * expert_output(t, k)) over valid routes,
 *                 +0 where a token has no valid route
 *   workspace     device scratch of at least w4a16_moe_workspace_size bytes;
 *                 its contents on entry do not matter and are clobbered.
 * The result does not depend on scheduling: every sum has a fixed order, so
 * repeated calls with the same inputs and variant give identical bits; the
 * fused finalize (descriptor) gives the same bits as the non-fused one, the
 * workgroup that combines a token being decided by integer arrival counters
 * in the workspace ([P2] Description: no atomic or reduction into the
 * output). */
w4a16_status_t w4a16_moe_forward(const void* x, const uint8_t* w13_packed,
                                 const void* w13_scales, const uint8_t* w2_packed,
                                 const void* w2_scales, const int32_t* topk_ids,
                                 const float* topk_weights, void* out,
                                 const w4a16_moe_desc_t* desc, void* workspace,
                                 size_t workspace_bytes, w4a16_stream_t stream);

/* w4a16_moe_forward, plus stage timing: stage_events[2*i] and
 * stage_events[2*i+1] (hipEvent_t created by the caller; null entries are
 * skipped) are recorded on `stream` right before and after stage i:
 *   i = 0 route preparation, 1 gate/up GEMM, 2 down GEMM (with the combine
 *   when it runs inside the down launch: the small-batch path, and the
 *   grouped path with fused_finalize = 1), 3 the combine launch (recorded
 *   back to back, empty, when the combine is fused).
 * n_events is the length of stage_events (0..8).  Same results as the
 * forward; meant for benchmarks. */
w4a16_status_t w4a16_moe_forward_timed(const void* x, const uint8_t* w13_packed,
                                       const void* w13_scales, const uint8_t* w2_packed,
                                       const void* w2_scales, const int32_t* topk_ids,
                                       const float* topk_weights, void* out,
                                       const w4a16_moe_desc_t* desc, void* workspace,
                                       size_t workspace_bytes, w4a16_stream_t stream,
                                       void* const* stage_events, int32_t n_events);

/* The forward with the router step fused in ([P2] Final performance: routing
 * is timed as part of the MoE; [P1] Benchmark: FP32 routing weights, INT32
 * ids, renormalization off in the measured workload).  Instead of ids and
 * weights it takes the router logits and routes every token inside the
 * forward's first launch (route preparation on the grouped path, the gate/up
 * GEMM on the small-batch path), as w4a16_moe_route_topk defines it (softmax
 * over all num_global_experts logits, the top_k largest in descending order,
 * ties to the lower id, optional renormalization), then runs the forward of
 * w4a16_moe_forward on those routes.
 *   router_logits [T][num_global_experts] fp32, device (num_global_experts of
 *                 the descriptor, 0 meaning num_local_experts; at most 1024,
 *                 and top_k at most 32 and at most num_global_experts)
 *   renormalize   0 or 1
 *   topk_ids      [T][K] int32 OUT: the routed global ids (ids outside the
 *                 local range are invalid routes of this share, as always)
 *   topk_weights  [T][K] fp32 OUT: their weights
 *   stage_events, n_events: as for w4a16_moe_forward_timed (NULL, 0 for none);
 *                 stage 0 is routing with route preparation, and on the
 *                 small-batch path stage 1 is routing with the gate/up GEMM.
 * Identical ids and weights to w4a16_moe_route_topk (same device code),
 * identical output bits to w4a16_moe_forward given those ids and weights.
 * Routing runs inside the first launch for up to 16 tokens on the grouped
 * path and up to 16 routes on the small-batch path (one token per wave);
 * beyond that the router runs as a launch of its own first (one wave per
 * token across the GPU is faster than several tokens per wave). */
w4a16_status_t w4a16_moe_forward_routed(const void* x, const uint8_t* w13_packed,
                                        const void* w13_scales, const uint8_t* w2_packed,
                                        const void* w2_scales, const float* router_logits,
                                        int32_t renormalize, int32_t* topk_ids,
                                        float* topk_weights, void* out,
                                        const w4a16_moe_desc_t* desc, void* workspace,
                                        size_t workspace_bytes, w4a16_stream_t stream,
                                        void* const* stage_events, int32_t n_events);

/* w4a16_moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, checks and results are those of
 * w4a16_moe_forward (same kernels, same plan, identical bits).  The scratch is
 * a library-owned device array of W4A16_NOALLOC_SCRATCH_BYTES (128 MiB) on each
 * GPU the library runs on, held until the process ends; its address is looked
 * up (not allocated) at the first call on a GPU, with the caller's current
 * device.  A descriptor whose workspace (w4a16_moe_workspace_size) exceeds it
 * is rejected with W4A16_ERR_UNSUPPORTED before anything is enqueued (the Kimi
 * shard shape fits up to about 960 tokens).  Every call on one GPU shares that
 * array and leaves its contents behind: calls on one GPU must be ordered (one
 * stream, or explicit dependencies); overlapping calls race and give wrong
 * results.  No hipMalloc, hipFree or other allocating call is made. */
#define W4A16_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
w4a16_status_t w4a16_moe_forward_noalloc(const void* x, const uint8_t* w13_packed,
                                         const void* w13_scales, const uint8_t* w2_packed,
                                         const void* w2_scales, const int32_t* topk_ids,
                                         const float* topk_weights, void* out,
                                         const w4a16_moe_desc_t* desc, w4a16_stream_t stream);

/* Route preparation alone, with the same device code the forward runs ([P1]
 * Benchmark, "route preparation"; [P2] Description, route guards and padded
 * fallback).  Uses desc->num_tokens, top_k, num_local_experts, expert_offset.
 *   counts        [E]     valid routes per local expert
 *   offsets       [E+1]   exclusive prefix sum of counts rounded up to
 *                         block_m (1..256); offsets[E] = padded total
 *   sorted_routes [sorted_capacity]  flat route index t*K+k of each padded
 *                         position, ascending within an expert; padding -1.
 *                         Positions at or past offsets[E] are not written.
 *   route_slot    [T*K]   position of each route in sorted_routes, or -1
 *   chunk_scratch NULL, or W4A16_ROUTE_CHUNKS_MAX * E int32 of device scratch
 *                 (contents on entry do not matter): with it the routes are
 *                 ranked in up to W4A16_ROUTE_CHUNKS_MAX chunks in parallel, as
 *                 in the forward; without it in one chunk.  Same results.
 *   sorted_capacity must be >= T*K + min(E, T*K) * (block_m - 1). */
#define W4A16_ROUTE_CHUNKS_MAX 32
w4a16_status_t w4a16_moe_prepare_routes(const w4a16_moe_desc_t* desc, const int32_t* topk_ids,
                                        int32_t block_m, int32_t* counts, int32_t* offsets,
                                        int32_t* sorted_routes, int64_t sorted_capacity,
                                        int32_t* route_slot, int32_t* chunk_scratch,
                                        w4a16_stream_t stream);

/* Routing fused with route preparation alone, with the device code of
 * w4a16_moe_forward_routed's grouped path ([P2] Final performance, routing
 * timed with the MoE): w4a16_moe_route_topk's ids and weights written to
 * topk_ids / topk_weights, and the tables of w4a16_moe_prepare_routes (same
 * arguments and meaning) built from them.  Uses desc->num_tokens, top_k,
 * num_local_experts, expert_offset and num_global_experts. */
w4a16_status_t w4a16_moe_route_and_prepare(const w4a16_moe_desc_t* desc,
                                           const float* router_logits, int32_t renormalize,
                                           int32_t block_m, int32_t* topk_ids,
                                           float* topk_weights, int32_t* counts,
                                           int32_t* offsets, int32_t* sorted_routes,
                                           int64_t sorted_capacity, int32_t* route_slot,
                                           int32_t* chunk_scratch, w4a16_stream_t stream);

/* Setup-time conversion of MXFP4 block scales (E8M0 codes e, value
 * 2^(e - 127); OCP microscaling formats) to the 16-bit scales the
 * FP4_GROUP_K layout takes (dtype W4A16_DT_BF16 or W4A16_DT_FP16; [P2] Final
 * performance: FP4 weights, weight preparation outside the timed region).
 *   e8m0   device, n codes
 *   out    device, n 16-bit values; exact for every code in bf16 except 255
 *          (NaN), in fp16 for 103 <= e <= 142
 * A code that has no exact 16-bit value writes the nearest one (NaN for 255);
 * n = 0 enqueues nothing. */
w4a16_status_t w4a16_e8m0_to_scales(const uint8_t* e8m0, int64_t n, int32_t dtype, void* out,
                                    w4a16_stream_t stream);

/* Setup-only re-layout of per-channel INT4 weights into the GROUP_K layout
 * ([P1] SGLang Marlin comparison: weight repacking is setup-only and outside
 * the timed region; [P3] Checkpoint format for the per-channel input).  The
 * values move from packing along the output dim to packing along K, and the
 * output channel's scale is repeated for each 32-value group of its row, so
 * every weight q[n][k] * s[n] is unchanged and the forward runs the group
 * layout's kernels on the result (qlayout W4A16_Q_GROUP_K, group 32).
 *   packed      [n_experts][n_out/2][k_in] u8 (PER_CHANNEL)
 *   scales      [n_experts][n_out] 16-bit
 *   out_packed  [n_experts][n_out][k_in/2] u8, 4-byte aligned (same size)
 *   out_scales  [n_experts][n_out][k_in/32] 16-bit (k_in/32 times as many)
 * n_out even, k_in a multiple of 64.  Bit-exact data movement. */
w4a16_status_t w4a16_repack_per_channel(const uint8_t* packed, const void* scales,
                                        int64_t n_experts, int32_t n_out, int32_t k_in,
                                        uint8_t* out_packed, void* out_scales,
                                        w4a16_stream_t stream);

/* Nibble unpacking with the device conversion the GEMMs use ([P3] Checkpoint
 * format): out[2i] = low nibble of packed[i], out[2i+1] = high nibble, both as
 * two's-complement int8 in [-8, 7].  out holds 2*n_bytes int8. */
w4a16_status_t w4a16_unpack_int4(const uint8_t* packed, int64_t n_bytes, int8_t* out,
                                 w4a16_stream_t stream);

/* FP4 (E2M1) decoding with the device conversion the GEMMs use ([P2]
 * Description, "Tests": the W4A4 cases kept beside W4A16; the element format
 * of the OCP microscaling specification): out[2i] = value of the low nibble
 * of packed[i], out[2i+1] = of the high nibble, as FP32 (exact: 0, +-0.5,
 * +-1, +-1.5, +-2, +-3, +-4, +-6, the sign of zero kept), the values passing
 * through the dtype's 16-bit form (dtype W4A16_DT_BF16 or W4A16_DT_FP16).
 * out holds 2*n_bytes floats; n_bytes = 0 enqueues nothing.  Errors:
 * W4A16_ERR_INVALID_ARG (negative size, unknown dtype, null pointer),
 * W4A16_ERR_UNSUPPORTED (n_bytes above 2^33). */
w4a16_status_t w4a16_decode_fp4(const uint8_t* packed, int64_t n_bytes, int32_t dtype, float* out,
                                w4a16_stream_t stream);

/* Router scoring and top-k, the step before route preparation ([P2] Final
 * performance: routing is timed with the MoE; [P1] Benchmark: FP32 routing
 * weights, INT32 ids, no renormalization).  For each token t:
 *   p_e = exp(l_e - max_j l_j) / sum_j exp(l_j - max_j l_j) over all
 *   num_global_experts logits (FP32), then the top_k experts of largest p in
 *   descending order, ties to the lower id; a logit of -inf has p = 0.
 *   logits        [T][num_global_experts] fp32, device, row-major
 *   topk_ids      [T][top_k] int32 out: global expert ids (feed
 *                 w4a16_moe_forward, which masks ids outside its local range)
 *   topk_weights  [T][top_k] fp32 out: p of each chosen expert, or p divided
 *                 by the sum of the top_k p (in top-k order) if renormalize = 1
 * Supported: 1 <= num_global_experts <= 1024, 1 <= top_k <= min(32,
 * num_global_experts), 0 <= num_tokens <= 2^31 - 1.  T = 0 enqueues nothing.
 * Errors are returned before anything is enqueued; NaN logits give an
 * unspecified selection.  Results are bitwise repeatable. */
w4a16_status_t w4a16_moe_route_topk(const float* logits, int64_t num_tokens,
                                    int32_t num_global_experts, int32_t top_k,
                                    int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                                    w4a16_stream_t stream);

/* Streaming-read probe (a measurement aid, not part of the forward): reads
 * the first (bytes / row_bytes) * row_bytes bytes of `buf` once, with the
 * access shape of the packed-weight stream (16 rows x 64 bytes per wave load
 * instruction, rows of row_bytes, the 8 waves of a workgroup splitting each
 * 16-row band), so that its time beside the forward's gives the achievable
 * HBM read rate for the weight bytes a forward streams ([P2] Final
 * performance times on cold caches; the weight stream is the roofline).
 *   buf       device, 16-byte aligned, at least `bytes` long
 *   row_bytes a multiple of 64, at most 8192
 *   sink      device uint32; written only for one improbable data value
 * Errors are returned before anything is enqueued. */
w4a16_status_t w4a16_stream_probe(const uint8_t* buf, int64_t bytes, int32_t row_bytes,
                                  uint32_t* sink, w4a16_stream_t stream);

/* Static text for a status code (unsupported configurations are strict
 * errors, not silent fallbacks: [P1] BC-breaking).  Never null; an unknown
 * code gives "unknown status". */
const char* w4a16_status_string(w4a16_status_t status);

/* Thread-local text of the last rejected call on this thread ("" if none):
 * the diagnostic names the offending tensor or descriptor field and the
 * value that failed, instead of a bare assertion ([P3] Description, the
 * alignment and shape diagnostics).  Owned by the library; valid until the
 * next call on the same thread. */
const char* w4a16_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_MOE_H */
