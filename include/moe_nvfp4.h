/*
 * moe_nvfp4.h -- C ABI of the weight-only NVFP4 fused MoE layer for AMD MI355X (gfx950).
 *
 * The layer (one pass per call of moe_nvfp4_forward):
 *   S1  router logits   logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e])        (fp32)
 *   S2  top-k           the k largest logits per token, descending, equal logits -> lower
 *                       expert index; weights = softmax over all E renormalised over the
 *                       k selected, i.e. exp(l_j - l_max) / sum_selected exp(l_i - l_max)
 *   S3  permute         group the T*k slots (slot = t*k + j) by expert, stable in slot order
 *   S4  gate/up GEMM    per expert e and row r of its group:
 *                       g = d_g * (x_t . Qg^T), u = d_u * (x_t . Qu^T), h = silu(g) * u
 *   S5  down GEMM       y_r = d_d * (h_r . Qd^T)
 *   S6  combine         out[t] = sum_j w[t][j] * y[row of slot t*k+j] + y_shared[t]
 * plus one always-on shared expert (weight 1, no gate) computed on every token.
 *
 * Sources (web pages; section names as printed there):
 *   - "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 6.1 "NVFP4 format":
 *     E2M1 elements (2-bit exponent, 1-bit mantissa, max 6.0) packed two per byte, one FP8 E4M3
 *     block scale per 16 contiguous elements along K, one fp32 global scale per tensor; an
 *     element's value is element * block scale * global scale.
 *   - same page, section 7.1: the modular fused-MoE stages Router -> Quantize-Dispatch ->
 *     Permute-Experts-Unpermute -> Combine; section 4 (b12x fused MoE): token dispatch, two
 *     GEMMs, SwiGLU and the top-k-weight reduction; section 5 (Marlin): weight-only W4A16,
 *     16-bit activations, weights dequantized to 16-bit inside the GEMM.
 *   - "Serving Solar Open 2 on DGX Spark": 320 routed experts + 1 shared expert, top-8
 *     ("Solar Open 2 in brief"); a shared module-level workspace pool instead of per-layer
 *     scratch, and fused gate/up projection ordering ("The fix" / "Supporting real NVFP4
 *     checkpoints").
 *   - "GLM-5.3-Flash-NVFP4 deployment blocked on SM121" (discussion): weight-only NVFP4 is
 *     selected by the absence of input quantization; a missing activation scale must never
 *     turn an expert's alpha into zero (MoE fault analysis); ModelOpt stores the dequant global
 *     scale amax/(448*6), compressed-tensors the quant scale (448*6)/amax (follow-up reply).
 *
 * Layout conventions (readings of the pages where they are silent):
 *   - bf16 values travel as uint16_t bit patterns.
 *   - A packed NVFP4 tensor [N][K] is N rows of K/2 bytes; element 2j of a row is the low nibble
 *     of byte j, element 2j+1 the high nibble; the nibble's top bit is the sign.
 *   - Its block scales are [N][K/16] E4M3FN bytes (bias 7, max 448, no infinities).
 *   - Fused gate/up weights w13 are [2I][H]: rows 0..I-1 gate, rows I..2I-1 up, each half with its
 *     own dequant global scale.
 *   - Checkpoints use the canonical layout above; the GEMM entry points read the weights after a
 *     one-time repack into the MFMA tile layout (moe_nvfp4_pack_tiles).
 *   - There is no activation-scale argument anywhere (W4A16): nothing can zero an expert.
 *
 * Conventions of every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  All buffers are owned by the caller; the
 *     library never allocates, frees or keeps a pointer after the call returns.
 *   - Activation, weight, scale, output and workspace pointers must be 16-byte aligned (the
 *     kernels use 16-byte vector accesses); a misaligned one gives MOE_ERR_INVALID_ARGUMENT.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is only enqueued: no host
 *     synchronisation, no device-to-host copy, so calls can be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; on error nothing is
 *     enqueued and a status != MOE_OK is returned.  A device that is not gfx950 gives
 *     MOE_ERR_UNSUPPORTED_DEVICE.  Launch failures give MOE_ERR_HIP.  Device faults surface at
 *     the caller's next synchronisation.  T == 0 is a valid no-op.
 *   - Results are deterministic: no floating-point atomics; repeated calls are bitwise equal.
 *   - Non-finite inputs are not checked and propagate.
 *   - Calls on one stream are ordered; calls that overlap in time must use distinct outputs and
 *     workspaces.
 *
 * Size limits: 1 <= k <= min(E, 64), E <= 1024; H and I multiples of 128 (the format needs 16;
 * the kernels' K-chunk is 128); T*k < 2^31; activation matrices (x: T*H, h: (T*k+T)*I, and the
 * `a` of a grouped GEMM: M_total*K, with every row it reads) under 4 GiB of bf16, since the
 * kernels that stage activation tiles address rows with 32-bit byte offsets.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED_DEVICE = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

/* Static, human-readable name of a status code (host). */
const char* moe_status_string(moe_status_t s);

/* Weight formats of an expert bank.  Both store E2M1 elements two per byte (element 2j in the low
 * nibble of byte j) and one block scale per group of consecutive elements along K:
 *   MOE_WEIGHT_NVFP4: E4M3FN scale per 16 elements and an fp32 global scale per tensor
 *                     ("vLLM on the NVIDIA DGX Spark", section 6.1);
 *   MOE_WEIGHT_MXFP4: E8M0 scale per 32 elements, value 2^(byte - 127) (0xFF NaN), no global scale
 *                     (same guide, section 6.4 "NVFP4 vs MXFP4"). */
#define MOE_WEIGHT_NVFP4 0
#define MOE_WEIGHT_MXFP4 1
/* MXFP4 weights in the W4A4 tile layout of moe_mxfp4_pack_tiles_a4: accepted only by the W4A4 entry
 * points (moe_mxfp4_w4a4_*), which in turn accept no other format, so a bank packed for one kernel
 * family can never be read by the other. */
#define MOE_WEIGHT_MXFP4_A4 2

/* One bank of experts (routed: num_experts = E; shared: num_experts = 1), device pointers.
 * The packed weights and block scales are in the MFMA TILE LAYOUT produced by
 * moe_nvfp4_pack_tiles (NVFP4), moe_mxfp4_pack_tiles (MXFP4) or moe_mxfp4_pack_tiles_a4 (MXFP4_A4)
 * from the canonical layout: per expert, the canonical [2I][H/2] (w13) or [H][I/2] (w2) bytes and
 * their scale bytes, permuted tile by tile (same sizes).  A zero-initialised `format` is NVFP4; the
 * routed and shared banks of a layer must share one format. */
typedef struct {
  int32_t num_experts;
  int32_t hidden;            /* H */
  int32_t inter;             /* I */
  int32_t format;            /* MOE_WEIGHT_NVFP4, MOE_WEIGHT_MXFP4 or MOE_WEIGHT_MXFP4_A4 */
  const uint8_t* w13;        /* [E] x tiled [2I][H/2]  packed E2M1, gate rows then up rows */
  const uint8_t* w13_scale;  /* [E] x tiled [2I][H/16] E4M3FN (NVFP4) or [2I][H/32] E8M0 (MXFP4) */
  const float* w13_gscale;   /* [E][2] dequant global scales (gate, up); NVFP4 only, may be NULL for MXFP4 */
  const uint8_t* w2;         /* [E] x tiled [H][I/2] */
  const uint8_t* w2_scale;   /* [E] x tiled [H][I/16] (NVFP4) or [H][I/32] (MXFP4) */
  const float* w2_gscale;    /* [E]; NVFP4 only, may be NULL for MXFP4 */
} moe_nvfp4_experts_t;

/* The whole layer: router + routed bank + optional shared bank (shared.num_experts == 0: none).
 * h16_norm (host values, NVFP4): bounds on the Euclidean norm of every dequantized gate row
 * (h16_norm[0]) and up row (h16_norm[1]) of both banks, global scales included, as
 * moe_nvfp4_h16_bound computes them.  Given (both finite and > 0), the W4A16 forward on 128-row
 * tiles holds h as fp16 rows scaled by a power of two per token chosen from these bounds, and runs
 * the down GEMM on fp16 operands too; zero (a zero-initialised struct): h stays bf16.  The result
 * is the same (bitwise, in practice) as long as the bounds hold; values below the true norms can
 * make h overflow fp16.  Larger values are safe: they only narrow the range below the bound in
 * which h is exact (2^31, see moe_nvfp4_forward). */
typedef struct {
  int32_t hidden;            /* H */
  int32_t num_experts;       /* E (routed) */
  int32_t top_k;             /* k */
  const uint16_t* w_router;  /* [E][H] bf16 */
  const float* router_bias;  /* [E] fp32 added to the logits, or NULL */
  moe_nvfp4_experts_t routed;
  moe_nvfp4_experts_t shared;
  float h16_norm[2];         /* gate, up; {0, 0}: off */
} moe_nvfp4_layer_t;

/* ---------------------------------------------------------------- S1 + S2: route
 * x [T][H] bf16, w_router [E][H] bf16, router_bias [E] fp32 or NULL.
 * Writes logits [T][E] fp32 (the router GEMM output, fp32 accumulation of exact bf16 products),
 * topk_ids [T][k] int32 (descending logit; equal logits -> lower index) and topk_w [T][k] fp32.
 * flags & MOE_ROUTE_LOGITS_GIVEN: skip the GEMM and select from the logits the caller passes in
 * `logits` (x, w_router and router_bias are then ignored and may be NULL).
 * Source: modular fused-MoE stages ("vLLM on the NVIDIA DGX Spark", section 7.1); top-8 of 320
 * ("Serving Solar Open 2 on DGX Spark", "Solar Open 2 in brief"). */
#define MOE_ROUTE_LOGITS_GIVEN 1u
moe_status_t moe_route(const uint16_t* x, const uint16_t* w_router, const float* router_bias,
                       int32_t T, int32_t H, int32_t E, int32_t k, uint32_t flags,
                       float* logits, int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------- S3: permute
 * topk_ids [T][k] int32 in [0, E).  Writes expert_counts [E], expert_offsets [E+1] (exclusive
 * prefix sum; offsets[E] = T*k), sorted_slot [T*k] (slot ids t*k+j grouped by expert, ascending
 * inside a group) and slot_to_row [T*k] (inverse permutation).  Bit-exact and atomic-order free.
 * Needs moe_permute_workspace_size(T, k, E) bytes of workspace.
 * Out-of-range ids (checked on the device; the route stage never produces them): a slot whose id is
 * outside [0, E) joins no group and nothing is written outside the output buffers.  Its slot_to_row
 * entry is -1, the counts and offsets leave it out, so expert_offsets[E] < T*k -- the caller's
 * signal that the ids were bad; sorted_slot entries at and past expert_offsets[E] are unspecified.
 * moe_combine turns every token holding such a slot into a NaN row.  The GEMM entry points, given
 * these offsets and M_total = T*k, leave output rows past expert_offsets[E] unwritten.
 * Source: "Permute-Experts-Unpermute" ("vLLM on the NVIDIA DGX Spark", section 7.1). */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);
moe_status_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* sorted_slot, int32_t* slot_to_row,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- S4 / S5: grouped NVFP4 GEMM
 * Rows [expert_offsets[e], expert_offsets[e+1]) of the M_total output rows use expert e of `w`
 * (expert_offsets: device [w->num_experts + 1], with expert_offsets[E] == M_total).
 *   MOE_GEMM_GATE_UP: A row r = a[row_index[r] / row_divisor] (or a[r] when row_index == NULL),
 *                     a has H columns; out[r] = bf16(silu(d_g * A_r.Qg^T) * (d_u * A_r.Qu^T)),
 *                     out is [M_total][I] bf16.
 *   MOE_GEMM_DOWN:    A row r = a[r] (row_index must be NULL), a has I columns;
 *                     out[r] = bf16(d_d * A_r.Qd^T), out is [M_total][H] bf16.
 * Weights are dequantized to bf16 (element * block scale is exact in bf16) and multiplied on the
 * bf16 matrix cores with fp32 accumulation; the fp32 global scale is applied to the accumulator.
 * Source: W4A16 "dequantize to 16-bit inside the GEMM" ("vLLM on the NVIDIA DGX Spark", section 5);
 * SiLU(gate)*up between the GEMMs (section 4, fused MoE); NVFP4 format (section 6.1). */
#define MOE_GEMM_GATE_UP 0
#define MOE_GEMM_DOWN 1
moe_status_t moe_nvfp4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w /* host */,
                                    const uint16_t* a, const int32_t* row_index, int32_t row_divisor,
                                    const int32_t* expert_offsets, int32_t M_total,
                                    uint16_t* out, void* stream);

/* ---------------------------------------------------------------- S6: combine
 * out[t][:] = bf16( sum_j topk_w[t][j] * y_rows[slot_to_row[t*k+j]][:] + y_shared[t][:] ),
 * accumulated in fp32 in the order j = 0..k-1, then the shared row.  y_shared may be NULL.
 * A negative slot_to_row entry (a slot moe_permute placed nowhere) is not read: the token's output
 * row is written as NaN.  Non-negative rows must lie inside y_rows (not checked).
 * Source: top-k-weight reduction of the fused MoE ("vLLM on the NVIDIA DGX Spark", section 4);
 * the shared expert is added with weight 1 ("Serving Solar Open 2 on DGX Spark": one shared
 * expert that every token uses). */
moe_status_t moe_combine(const uint16_t* y_rows, const int32_t* slot_to_row, const float* topk_w,
                         const uint16_t* y_shared, int32_t T, int32_t k, int32_t H,
                         uint16_t* out, void* stream);

/* ---------------------------------------------------------------- whole layer
 * Optional extra outputs of moe_nvfp4_forward (each may be NULL): the router logits [T][E],
 * the selection topk_ids [T][k], topk_w [T][k], and expert_counts [E] (device pointers).
 * stage_events (host array of MOE_NUM_STAGE_EVENTS hipEvent_t handles, or NULL): when given,
 * event i is recorded on the stream at stage boundary i -- 0 before S1, 1 after S1, 2 after S2+S3,
 * 3 after S4, 4 after S5, 5 after S6 -- so callers can time each stage; NULL entries are skipped.
 * Where S4's GEMM reads x as fp16 rows (NVFP4 on 128-row tiles), event 2 follows the pass that
 * writes them, so that the S4 interval holds the GEMM launches alone.
 * The events are created and owned by the caller.
 * y_rows (device, bf16 [T*k + T_shared][H], T_shared = T with a shared expert, else 0): when given,
 * the expert outputs of S5 are written there instead of the workspace -- row r < T*k is the routed
 * expert output of sorted row r (slot sorted_slot[r] of the permutation), row T*k + t the shared
 * expert's output for token t -- the inputs of the combine, for callers that check the stages.
 * flags: MOE_FORWARD_FUSED_DECODE runs the two-launch fused decode path below where it applies
 * (elsewhere the flag is ignored); both paths compute bitwise the same output.
 *
 * Fused decode path (opt-in): with few tokens (T <= 32, T*k <= 256, E <= 320, NVFP4 banks, a shared
 * expert of the routed width or none, at most 8 rows per expert on average) the forward is two
 * launches: the router, then S2-S6 in one kernel whose workgroups hand work on through counters in
 * the workspace (cleared by the router launch; every wait points at a workgroup of smaller index and
 * is bounded: past the bound the output rows are NaN).  Its stage events 2, 3 and 4 are recorded
 * after that second launch, with event 5.  On MI355X it is slower than the staged launches (the
 * completion counters of the gate/up tiles become visible to the waiting down tiles tens of
 * microseconds late while the weights stream at full bandwidth), so it is not the default.  Source:
 * the fused MoE kernel (token dispatch, two GEMMs, SwiGLU, top-k-weight reduction in one launch;
 * "vLLM on the NVIDIA DGX Spark", section 4) and the separate small-batch micro path ("Serving Solar
 * Open 2 on DGX Spark", "Adding Expert Parallelism to b12x"). */
#define MOE_NUM_STAGE_EVENTS 6
#define MOE_FORWARD_FUSED_DECODE 1u
typedef struct {
  float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_counts;
  void* const* stage_events;
  uint16_t* y_rows;
  uint32_t flags;
} moe_forward_aux_t;

/* Workspace bytes moe_nvfp4_forward needs for T tokens (I_shared = 0: no shared expert).  It holds
 * the router logits (and, for a router GEMM split along K, up to three more [T][E] fp32 arrays of
 * partial sums), the selection, the permutation, x as fp16 rows with one power-of-two shift
 * per row ([T][H] fp16 + [T] int32; read by the NVFP4 gate/up GEMM on prefill shapes, an exact
 * re-encoding of the bf16 values), the intermediate h (row-major, or in the 128-row-tile fragment
 * order the prefill-shaped GEMMs exchange it in: up to (min(E, T*k) + T*k/128 + ceil(T/128)) * 128
 * rows), one int32 power of two per h row ((T*k + T) when h takes the tile order) and the expert
 * outputs y [(T*k + T)][H]. */
size_t moe_nvfp4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared,
                                        int32_t E, int32_t k);

/* S1..S6 for x [T][H] bf16 -> out [T][H] bf16.  `layer` and `aux` are host pointers to structs
 * holding device pointers.  The workspace may be shared by every layer of a model that runs on
 * the same stream (one pool instead of per-layer scratch).  On 128-row tiles with layer->h16_norm
 * given, h = bf16(silu(g) * u) enters the down GEMM as fp16 after scaling by 2^hs per token, with
 * hs chosen so that the bound ||x||^2 h16_norm[0] h16_norm[1] on |h| (|silu(g)| <= |g|) lands below
 * 2^14: every h within 2^31 of that bound is carried exactly (the down sums are then those of the
 * bf16 h), smaller ones round to the fp16 subnormal grid (absolute error below 2^-38 of the bound). */
moe_status_t moe_nvfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                               uint16_t* out, void* workspace, size_t workspace_bytes,
                               const moe_forward_aux_t* aux, void* stream);

/* The whole layer for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, hosts that forbid hipMalloc): moe_nvfp4_forward with its workspace in a device array the
 * library holds, MOE_NOALLOC_SCRATCH_BYTES on every GPU it runs on, until the process ends.  No
 * allocation, no free, no memset.  A layer and T whose moe_nvfp4_forward_workspace_size exceeds
 * the array give MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (64 MiB covers T up to
 * about 580 tokens at H=4096, I=1536, E=320, k=8 with a shared expert).  All calls on one GPU share
 * its array and it keeps the last call's contents: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  Arguments otherwise as for
 * moe_nvfp4_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_nvfp4_forward_noalloc(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                                       uint16_t* out, const moe_forward_aux_t* aux, void* stream);

/* Pure-host validation used by moe_nvfp4_forward; needs no GPU when gfx_arch is given
 * (e.g. "gfx950"; NULL = query the current device). */
moe_status_t moe_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                  const char* gfx_arch);

/* ---------------------------------------------------------------- weight preparation
 * Load-time conversion of compressed-tensors global scales (host memory): the checkpoint stores
 * the quant scale q = (448*6)/amax, the kernels take the dequant scale d = fp32(1/q).
 * Source: the reciprocal between ModelOpt and compressed-tensors global scales ("GLM-5.3-Flash-
 * NVFP4" discussion, compressed-tensors follow-up).  Fails on q == 0 or non-finite q. */
moe_status_t moe_gscale_from_quant_scale(const float* q_host, float* d_host, int32_t n);

/* Load-time repack of canonical NVFP4 tensors into the MFMA tile layout every GEMM entry point
 * reads.  Input: num_tensors tensors of [rows][cols] weights as canonical packed bytes
 * [rows][cols/2] and scale bytes [rows][cols/16] (rows % 16 == 0, cols % 128 == 0).  Output (same
 * sizes, out of place): tile t = (rows/16 block nb) * (cols/128) + (128-column chunk c) of each
 * tensor holds 1024 nibble bytes and 128 scale bytes.  With l = 16q + n (q, n in 0..3, 0..15) and
 * j in 0..3, nibble bytes [16l + 4j, 16l + 4j + 4) are canonical bytes [64c + 16j + 4q, +4) of row
 * 16nb + n (the elements [128c + 32j + 8q, +8)), and scale bytes [8n, 8n + 8) are that row's
 * canonical scale bytes 8c + {0, 2, 4, 6, 1, 3, 5, 7}.  A fused gate/up tensor of one expert is one
 * [2I][H] tensor.  One wave then reads a whole tile with one contiguous 1 KB load, each lane
 * holding the operand of four 16x16x32 MFMA steps.
 * Source: the checkpoint-preparation step that swizzles weights into a kernel's MMA tile layout
 * ("Serving Solar Open 2 on DGX Spark", "Supporting real NVFP4 checkpoints"). */
moe_status_t moe_nvfp4_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream);

/* Load time, NVFP4: the bounds of moe_nvfp4_layer_t::h16_norm for one tiled bank.  For every expert e
 * and every gate row j (rows [0, I) of w13) the Euclidean norm of d_g[e] * e2m1(code) * e4m3(scale)
 * over the row's H elements (fp64, then rounded up to fp32), likewise for the up rows with d_u[e];
 * the largest gate-row norm and the largest up-row norm are folded into bound[0] and bound[1] with a
 * maximum.  bound: device, two floats, zero-filled by the caller once; call for the routed and the
 * shared bank of a layer, then copy bound to h16_norm.  An E4M3 NaN scale leaves a NaN bound (the
 * fp16 h path then stays off).  Errors: MOE_ERR_INVALID_ARGUMENT for a non-NVFP4 bank, a NULL
 * tensor, I % 16 or H % 128 nonzero.  Enqueued on `stream`.
 * Source: the fp32 global scale of each NVFP4 tensor and the E2M1 x E4M3 dequantization
 * ("vLLM on the NVIDIA DGX Spark", section 6.1). */
moe_status_t moe_nvfp4_h16_bound(const moe_nvfp4_experts_t* bank /* host */, float* bound, void* stream);

/* On-device NVFP4 quantization of fp32 weights (the on-the-fly quantization path a checkpoint
 * without pre-quantized weights needs).  w: num_tensors tensors of [rows][cols] fp32, contiguous;
 * gscale: device [num_tensors] dequant global scales d.  Per 16-group along cols, in fp32:
 *   s = E4M3_RNE(min(amax_group / (6*d), 448)),  code = E2M1_RNE(w / (s*d)) (saturating at 6;
 *   all codes 0 when s == 0; the sign bit is set for negative w).
 * Writes packed [num_tensors][rows][cols/2] and scales [num_tensors][rows][cols/16].
 * cols must be a multiple of 16.
 * Source: the recipe g16 / symmetric / tensor-group / FP8-E4M3 block scales ("GLM-5.3-Flash-NVFP4"
 * discussion); block scales clamped to 448 ("Serving Solar Open 2 on DGX Spark"). */
moe_status_t moe_nvfp4_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols,
                                const float* gscale, uint8_t* packed, uint8_t* scales, void* stream);

/* MXFP4 counterpart of moe_nvfp4_pack_tiles: canonical packed bytes [rows][cols/2] and E8M0 scale
 * bytes [rows][cols/32] (rows % 16 == 0, cols % 128 == 0) -> tiles of 1024 nibble bytes (the NVFP4
 * nibble permutation) and 64 scale bytes: bytes [4n, 4n + 4) of tile t are the canonical scale
 * bytes [4c, 4c + 4) of row 16nb + n, so byte j is the scale of the elements [128c + 32j, +32),
 * the operand of MFMA step j.  Same sizes as the canonical layout; out of place.
 * Source: MXFP4 format ("vLLM on the NVIDIA DGX Spark", section 6.4); the one-time swizzle into
 * the kernel's MMA layout ("Serving Solar Open 2 on DGX Spark", "Supporting real NVFP4
 * checkpoints"). */
moe_status_t moe_mxfp4_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream);

/* On-device MXFP4 quantization of fp32 weights (test and checkpoint-conversion data, not part of
 * the layer pass).  w: num_tensors tensors of [rows][cols] fp32.  Per 32-group along cols:
 *   e = floor(log2(amax_group)) - 2 clamped to [-127, 127] (-127 when amax == 0), scale byte e + 127;
 *   code = E2M1_RNE(|w| * 2^-e) saturating at 6, sign bit set for negative w.
 * Writes packed [num_tensors][rows][cols/2] and scales [num_tensors][rows][cols/32]; cols % 32 == 0.
 * Source: MXFP4 format (section 6.4 of the guide above); the shared-exponent rule is the OCP
 * Microscaling conversion (the guide does not state one). */
moe_status_t moe_mxfp4_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols, uint8_t* packed,
                                uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- W4A4 (MXFP4 weights and activations)
 * The W4A4 variant of the layer: the activations entering each GEMM are quantized to 4 bits as
 * well and the GEMMs run on the FP4 matrix cores (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4), both
 * operands in the MXFP4 format (E2M1 elements, one E8M0 scale per 32 elements along K).
 * Source: W4A4 checkpoints carry 4-bit weights and activations and run a native FP4 matmul, whose
 * gain is in prefill ("vLLM on the DGX Spark, the Hard Way: Seven Months of GB10 Field Notes",
 * "The one rule that explains all the FP4 confusion" and "Measured: native FP4 + MTP vs the
 * published Marlin numbers"); the fused MoE kernel quantizes bf16 hidden states to FP4 itself
 * ("vLLM on the NVIDIA DGX Spark", section 4.3); MXFP4 (same guide, section 6.4).  The pages'
 * NVFP4 activation format (E4M3 per 16 elements plus a global scale) has no counterpart in the
 * gfx950 FP4 instruction, whose block scales are E8M0 per 32 elements, so both sides use MXFP4.
 *
 * MXFP4 quantization of bf16 rows: a [rows][cols] bf16 -> packed [rows][cols/2] E2M1 codes and
 * scales [rows][cols/32] E8M0, per 32-group by the rule of moe_mxfp4_quantize (computed exactly on
 * the bf16 values).  cols % 32 == 0; a and packed 16-byte aligned. */
moe_status_t moe_mxfp4_quantize_act(const uint16_t* a, int32_t rows, int32_t cols, uint8_t* packed,
                                    uint8_t* scales, void* stream);

/* Load-time repack of canonical MXFP4 tensors into the W4A4 tile layout the W4A4 GEMMs read:
 * tile t = (rows/16 block nb) * (cols/128) + (128-column chunk c) holds 1024 nibble bytes and 64
 * scale bytes; with l = 16q + n, nibble bytes [16l, 16l + 16) are the canonical bytes
 * [64c + 16q, +16) of row 16nb + n (its elements [128c + 32q, +32), one scale block) and scale
 * byte l is that row's canonical scale byte 4c + q.  rows % 16 == 0, cols % 128 == 0; out of
 * place, same sizes.  A bank for the W4A4 entry points has format MOE_WEIGHT_MXFP4_A4 and its
 * weights in this layout (not the one of moe_mxfp4_pack_tiles). */
moe_status_t moe_mxfp4_pack_tiles_a4(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                     int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream);

/* W4A4 grouped GEMM, the counterpart of moe_nvfp4_grouped_gemm: A row r is MXFP4 activation row
 * a[row_index[r] / row_divisor] (or a[r]) -- codes `a` [rows][K/2], scales `a_scale` [rows][K/32]
 * from moe_mxfp4_quantize_act -- and every product of a weight and an activation is exact before
 * the fp32 accumulation.  Gate/up writes h = bf16(silu(A.Qg^T) * (A.Qu^T)) [M_total][I]; down
 * writes y = bf16(A.Qd^T) [M_total][H].  w->format must be MOE_WEIGHT_MXFP4_A4 (W4A4 tile layout);
 * a, a_scale and out 16-byte aligned; M_total * K / 2 < 4 GiB. */
moe_status_t moe_mxfp4_w4a4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w, const uint8_t* a,
                                         const uint8_t* a_scale, const int32_t* row_index, int32_t row_divisor,
                                         const int32_t* expert_offsets, int32_t M_total, uint16_t* out,
                                         void* stream);

/* Workspace bytes of moe_mxfp4_w4a4_forward: the routing buffers, x and h in MXFP4, h in bf16 and
 * the expert outputs y. */
size_t moe_mxfp4_w4a4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared,
                                             int32_t E, int32_t k);

/* Host validation of moe_mxfp4_w4a4_forward (as moe_validate_forward, plus MXFP4 banks). */
moe_status_t moe_mxfp4_w4a4_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                             const char* gfx_arch);

/* The W4A4 layer: S1-S3 and S6 as moe_nvfp4_forward; S4 quantizes x to MXFP4 (once per token) and
 * runs the W4A4 gate/up GEMM, S5 quantizes the bf16 h rows to MXFP4 and runs the W4A4 down GEMM.
 * Banks in the W4A4 tile layout; aux and stage events as for moe_nvfp4_forward. */
moe_status_t moe_mxfp4_w4a4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    const moe_forward_aux_t* aux, void* stream);

/* ---------------------------------------------------------------- W4A4 in NVFP4 (numerics)
 * The pages' own W4A4 method: NVFP4 weights (the W4A16 banks: format MOE_WEIGHT_NVFP4, tile layout
 * of moe_nvfp4_pack_tiles) times NVFP4 activations -- E2M1 elements, one E4M3 block scale per 16
 * elements along K and one fp32 global scale per GEMM input -- the two global scales combined as
 * alpha = 1 / (input_global_scale * weight_global_scale) in the GEMM epilogue ("vLLM on the NVIDIA
 * DGX Spark: A Complete Technical Guide", section 6.1; the fused MoE quantizes its bf16 inputs to
 * FP4 itself, section 4.3 and the table of section 4.5).  Global scales are taken in dequant form
 * d (the ModelOpt convention; a compressed-tensors quant scale is 1 / d), so alpha = d_act * d_w.
 * One static (calibrated) activation scale per GEMM input, shared by every expert: act_gscale_x
 * for the gate/up input x, act_gscale_h for the down input h, which is rounded to bf16 first.
 * A zero, negative or non-finite activation scale gives MOE_ERR_INVALID_ARGUMENT before anything
 * is enqueued: a missing activation scale folded into the alphas multiplies every expert by zero
 * ("GLM-5.3-Flash-NVFP4 deployment blocked on SM121" discussion).
 * The gfx950 FP4 matrix instruction takes E8M0 scales per 32 elements only, so this path forms the
 * products exactly on 16-bit operands instead: the quantizer writes each activation as the bf16
 * value e2m1(code) * e4m3(block scale) -- at most 6 significant bits within [2^-10, 2688], exact --
 * and the W4A16 GEMMs run on those rows with alpha in their epilogue.  It is for numerics, not
 * speed: the W4A16 layer's time plus the two quantization passes.
 *
 * NVFP4 quantization of bf16 rows: a [rows][cols] -> packed [rows][cols/2] E2M1 codes (element 2j
 * in the low nibble of byte j), scales [rows][cols/16] E4M3 bytes and values [rows][cols] bf16
 * (e2m1 * e4m3, without the global scale), per 16-group by the rule of moe_nvfp4_quantize with the
 * dequant global scale `gscale` (every decision in fp32).  Each output may be NULL, not all
 * three; values may be a itself (in place).  cols % 16 == 0; a, packed and values 16-byte aligned;
 * gscale finite and positive. */
moe_status_t moe_nvfp4_quantize_act(const uint16_t* a, int32_t rows, int32_t cols, float gscale, uint8_t* packed,
                                    uint8_t* scales, uint16_t* values, void* stream);

/* W4A4 grouped GEMM in NVFP4: moe_nvfp4_grouped_gemm on A rows that hold the `values` of
 * moe_nvfp4_quantize_act, whose dequant global scale act_gscale the epilogue applies together
 * with the weight's (h or y = bf16 of the sums times d_act * d_w).  w->format must be
 * MOE_WEIGHT_NVFP4; act_gscale finite and positive; otherwise as moe_nvfp4_grouped_gemm. */
moe_status_t moe_nvfp4_w4a4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w, const uint16_t* a,
                                         float act_gscale, const int32_t* row_index, int32_t row_divisor,
                                         const int32_t* expert_offsets, int32_t M_total, uint16_t* out,
                                         void* stream);

/* Workspace bytes of moe_nvfp4_w4a4_forward: those of moe_nvfp4_forward plus x's 4-bit values
 * as bf16 rows [T][H]. */
size_t moe_nvfp4_w4a4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared,
                                             int32_t E, int32_t k);

/* Host validation of moe_nvfp4_w4a4_forward: as moe_validate_forward, plus NVFP4 banks and usable
 * activation scales. */
moe_status_t moe_nvfp4_w4a4_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                             float act_gscale_x, float act_gscale_h, const char* gfx_arch);

/* The NVFP4 W4A4 layer: S1-S3 and S6 as moe_nvfp4_forward (routing on the bf16 tokens); S4
 * quantizes x (once per token) and runs the gate/up GEMM on its 4-bit values, S5 quantizes the
 * bf16 h rows in place and runs the down GEMM on theirs.  aux and stage events as for
 * moe_nvfp4_forward (the fused-decode flag is ignored). */
moe_status_t moe_nvfp4_w4a4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                                    float act_gscale_x, float act_gscale_h, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, const moe_forward_aux_t* aux, void* stream);

/* ---------------------------------------------------------------- measurement helper
 * Not a step of the layer: reads `bytes` bytes of device memory at `buf` once with a plain
 * streaming-read kernel (16-byte non-temporal loads, at most `workgroups` workgroups of 256 threads
 * in a grid-stride loop) and writes nothing but, in a case that never arises for real data, one
 * word to `sink` (device, 4 bytes).  Timed by the caller, it gives the HBM read bandwidth this GPU
 * reaches, the practical ceiling of the weight-stream-bound decode GEMMs (decode re-reads the active
 * weights for every token and is memory-bandwidth bound: "vLLM on the DGX Spark, the Hard Way: Seven
 * Months of GB10 Field Notes", "The five-minute model of what vLLM is doing on this box", item 1).
 * bytes % 16 == 0, buf 16-byte aligned, 1 <= workgroups <= 2^20. */
moe_status_t moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
