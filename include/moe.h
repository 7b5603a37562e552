/*
 * moe.h -- C ABI of libmoe.so: the routed Mixture-of-Experts FFN of a
 * DeepSeek-V4-Flash-shaped layer with block-quantized (MXFP4) experts,
 * computed by hand-written HIP kernels for gfx950 (MI355X).
 *
 * The method (pages cited by title):
 *   "DeepSeek-V4-Flash 284B (13.17B Active) -- Deep-Dive Mathematical &
 *   Kernel Guide" (llama-modchip):
 *     section 1: 256 routed experts + 1 shared, 6 active, routed scale 1.5;
 *       learned layers gate with SQRT_SOFTPLUS, hash layers look token ids up
 *       in a token-id -> 6-expert table (ffn_gate_tid2eid);
 *     section 3.2, MoE combine equation: y = e_shared(x) + sum_i w_i e_{k_i}(x),
 *       sum_i w_i = 1.5;
 *     section 4, SwiGLU equation: h = SiLU(W_gate x) * (W_up x), y = W_down h.
 *   "DeepSeek V4 target engine (CPU + optional CUDA tier)", introduction:
 *     routed experts in native fp4 (MXFP4), dense weights in fp8-e4m3 with
 *     UE8M0 block scales.
 *   "Development Snapshot Validation" (cism), 4-bit quantization scheme
 *     study: MXFP4 = E2M1 elements + one E8M0 scale per 32 elements.
 *
 * Conventions for every entry point
 *   - Array arguments are device pointers owned by the caller.  moe_layer
 *     itself is host memory that is read during the call only.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; 0 is the
 *     null stream); the caller synchronises.  Calls keep no state between
 *     them and allocate nothing; scratch memory comes from the caller's
 *     workspace, sized by the matching *_workspace_bytes query.
 *   - Host-checkable argument errors return MOE_ERR_INVALID,
 *     MOE_ERR_UNSUPPORTED or MOE_ERR_WORKSPACE before anything is enqueued.
 *     A failed kernel launch returns MOE_ERR_DEVICE.  Nothing is thrown.
 *   - Data errors found on the device (an expert id or token id out of
 *     range) are OR-ed into the optional `dev_error` word (never cleared by
 *     the library) with no host synchronisation; the offending entry is
 *     skipped and every access stays in bounds.
 *   - n_tokens == 0 is valid; moe_group (and moe_route_group) then write
 *     zero counts and offsets, every other call enqueues nothing.
 *
 * Weight layout (the pages print no layout; this is the reading used):
 *   A projection is a stack of experts, expert e at byte offset
 *   e * rows * row_bytes of `codes` (and likewise for `scales`).  Rows are
 *   output features; gate/up have rows = inter, cols = hidden; down has
 *   rows = hidden, cols = inter.
 *   MOE_W_MXFP4: codes uint8 [rows][cols/2]; byte b of a row holds element
 *     2b in bits 0..3 and element 2b+1 in bits 4..7; an element is an E2M1
 *     code (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
 *     0, .5, 1, 1.5, 2, 3, 4, 6).  scales uint8 [rows][cols/32]; scale j of
 *     a row is a UE8M0 byte u meaning 2^(u-127) for elements 32j..32j+31.
 *   MOE_W_FP8E4M3_B128: codes uint8 [rows][cols], OCP E4M3 ("fn": bias 7,
 *     max 448, no infinities); scales uint8 [rows][cols/128], one UE8M0 per
 *     128 elements of a row.
 *   The three routed matrices share one weight type, and so do the three
 *   shared ones (MOE_ERR_UNSUPPORTED otherwise).
 *   Decode is exact for scale bytes 2..252 (every element times its scale
 *   is then a normal bfloat16 number); other bytes are outside the
 *   supported range and give unspecified (but in-bounds) results.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* a null/misaligned pointer or an impossible size */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels cover    */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  MOE_ERR_DEVICE = 4       /* a HIP call or kernel launch failed              */
} moe_status;

typedef enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act_type;

typedef enum { MOE_W_MXFP4 = 0, MOE_W_FP8E4M3_B128 = 1 } moe_weight_type;

/* Bits OR-ed into dev_error. */
#define MOE_DEVERR_EXPERT_ID 1 /* an expert id outside [0, n_experts)  */
#define MOE_DEVERR_TOKEN_ID 2  /* a token id outside [0, vocab)        */
#define MOE_DEVERR_SYNC 4      /* moe_forward: a wait of the single-token kernel timed
                                  out (the rows of y it owned are NaN)  */

/* Limits of the library. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 8
#define MOE_MAX_DIM 65536
#define MOE_MAX_TOKENS (1 << 22)

typedef struct {
  int32_t type; /* moe_weight_type */
  const uint8_t* codes;  /* 16-byte aligned */
  const uint8_t* scales; /* 16-byte aligned */
} moe_proj;

typedef struct {
  int32_t hidden;    /* multiple of 128, <= MOE_MAX_DIM                  */
  int32_t inter;     /* routed expert intermediate size, multiple of 128 */
  int32_t n_experts; /* routed experts, 1..MOE_MAX_EXPERTS               */
  int32_t top_k;     /* 1..MOE_MAX_TOP_K, <= n_experts                   */
  moe_proj gate, up, down; /* routed, stacked over n_experts             */
  int32_t has_shared;      /* 0 or 1: one shared expert, weight 1        */
  int32_t shared_inter;    /* multiple of 128 when has_shared            */
  moe_proj shared_gate, shared_up, shared_down; /* one matrix each       */
  /* Optional (NULL: unused): the layer's weights as written by
   * moe_pack_experts, 256-byte aligned.  The batched gate/up and down read
   * them from there; every other path reads the arrays above, which stay
   * required and must hold the same weights. */
  const void* packed_experts;
} moe_layer;

/*
 * Options beyond the plain path, taken by the *_ex entry points (a NULL
 * pointer, or a zeroed struct, asks for none of them).  Host memory, read
 * during the call only.
 *
 * Group-limited selection ("Deep-Dive Mathematical & Kernel Guide", section
 * 1: SQRT_SOFTPLUS gating "with expert group top-k selection"; the pages
 * give no group parameters, this is the reading taken):
 *   n_group     experts form n_group contiguous groups of n_experts/n_group;
 *               0 or 1: one group.  At most 64, dividing n_experts.
 *   topk_group  a token takes its experts from the topk_group groups whose
 *               two largest selection keys sum highest (ties to the lower
 *               group); 0 means n_group.  topk_group * n_experts / n_group
 *               must be at least top_k.
 *   sel_bias    nullable device fp32 [n_experts]: the selection key of expert
 *               e is s_e + sel_bias[e] with s = sqrt(softplus(logit)) in fp64;
 *               the bias moves the selection only, the weights use s.
 *   With more than one group or a bias the top_k largest keys of the kept
 *   groups are chosen (ties to the lower expert index); without either the
 *   selection is moe_route's (on the logits).
 * Tail pruning with L2-quadrature rescaling (Guide section 3.2 item 3 and
 * its configuration table; "[RFC / Benchmarks] Fitting 284B
 * DeepSeek-V4-Flash in 57.61 GiB RAM", section 5):
 *   keep_max    at most this many routed experts per token (the largest
 *               weights, ties to the lower slot); 0 means top_k.
 *   min_w       routed experts whose weight is below min_w are dropped (the
 *               weights sum to routed_scale, so the RFC's p_early = 0.025
 *               is min_w = 0.025 * routed_scale); at least one expert (the
 *               largest weight) is always kept.  0: no threshold.
 *   Kept weights are multiplied by sqrt(sum of all w^2 / sum of kept w^2)
 *   (fp64 from the fp32 weights, rounded once); a dropped slot gets expert
 *   id -1 and weight 0 and keeps its position.  moe_group treats id -1 as
 *   "no expert", so the dropped experts' weights are never read.
 * Gate-first lazy skip (RFC section 5):
 *   lazy_tau    a routed expert whose gate output g for a token has
 *               max_j |SiLU(g_j)| < lazy_tau contributes nothing to that
 *               token; 0: off.  The shared expert is never skipped.  For
 *               bf16 batches of up to 16 tokens with MXFP4 experts the gate
 *               projection runs first and a skipped expert's up and down
 *               weights are not read (when all of its tokens skip it); other
 *               batches compute every expert and drop the skipped terms.
 */
typedef struct {
  int32_t n_group;
  int32_t topk_group;
  const float* sel_bias;
  int32_t keep_max;
  float min_w;
  float lazy_tau;
} moe_opts;

/*
 * Learned router ("Deep-Dive Mathematical & Kernel Guide", section 1,
 * gating_func SQRT_SOFTPLUS; section 3.2, sum of routed weights 1.5).
 *   logits     fp32 [n_tokens][n_experts], row-major, finite.
 *   topk_ids   out int32 [n_tokens][top_k]: the top_k largest logits of the
 *              token, slot 0 the largest, ties to the lower expert index
 *              (-0 equals +0).  The ids of a token are always distinct
 *              (non-finite logits give unspecified but distinct ids).
 *   topk_w     out fp32 [n_tokens][top_k]: s_i = sqrt(softplus(logit_i)),
 *              w_i = routed_scale * s_i / sum_j s_j (evaluated in fp64,
 *              rounded to fp32 once).
 *   Expert groups are read as a single group (plain top-k over all experts).
 */
moe_status moe_route(const float* logits, int n_tokens, int n_experts, int top_k,
                     float routed_scale, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream);

/* moe_route with the routing options of moe_opts (groups, selection bias,
 * tail pruning; lazy_tau is not a routing option and is ignored here).
 * MOE_ERR_INVALID for options outside the ranges stated with moe_opts. */
moe_status moe_route_ex(const float* logits, int n_tokens, int n_experts, int top_k,
                        float routed_scale, const moe_opts* opts, int32_t* topk_ids,
                        float* topk_w, hipStream_t stream);

/*
 * Token-id hash router ("Deep-Dive Mathematical & Kernel Guide", section 1
 * and section 3.2 item 1: ffn_gate_tid2eid maps a token id to 6 experts with
 * flat weights).
 *   token_ids  int32 [n_tokens], each in [0, vocab).
 *   tid2eid    int32 [vocab][top_k] expert ids; tid2w fp32 [vocab][top_k].
 *   topk_ids / topk_w  out, [n_tokens][top_k]: the token's table row in table
 *              order.  A token id out of range gives ids -1 and weights 0
 *              and sets MOE_DEVERR_TOKEN_ID in *dev_error (dev_error may be
 *              NULL).
 */
moe_status moe_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                          const float* tid2w, int vocab, int n_experts, int top_k,
                          int32_t* topk_ids, float* topk_w, int32_t* dev_error,
                          hipStream_t stream);

/*
 * moe_route followed by moe_group on the same ids, with the same outputs
 * and rules as those two calls.  Batches with n_tokens*top_k <= 4096 run in
 * a single launch (one workgroup routes the tokens and groups them in LDS),
 * which matters when the batch is a few decode tokens; larger batches use
 * the two kernels.
 */
moe_status moe_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                           float routed_scale, int32_t* topk_ids, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int32_t* dev_error, hipStream_t stream);

/* moe_route_group with the routing options of moe_opts. */
moe_status moe_route_group_ex(const float* logits, int n_tokens, int n_experts, int top_k,
                              float routed_scale, const moe_opts* opts, int32_t* topk_ids,
                              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* dev_error, hipStream_t stream);

/* Workspace bytes moe_group needs (currently 0: it works in LDS). */
size_t moe_group_workspace_bytes(int n_tokens, int top_k, int n_experts);

/*
 * Token-to-expert grouping (the expert bucketing behind MUL_MAT_ID row-group
 * reuse, "Deep-Dive Mathematical & Kernel Guide" section 2 table A and
 * section 6 item 2).  With f = t*top_k + i the flat index of slot i of
 * token t:
 *   counts    out int32 [n_experts]: number of f with topk_ids[f] == e.
 *   offsets   out int32 [n_experts+1]: exclusive prefix of counts.
 *   perm      out int32 [n_tokens*top_k]: the flat indices sorted by expert,
 *             ascending f inside an expert (stable); only the first
 *             offsets[n_experts] entries are written.
 *   inv_perm  out int32 [n_tokens*top_k]: inv_perm[perm[p]] = p; -1 for an
 *             entry whose id is -1 (a slot dropped by tail pruning: it
 *             belongs to no expert and is not an error) or out of range (then
 *             MOE_DEVERR_EXPERT_ID is set in *dev_error; dev_error may be
 *             NULL).
 *   Results are deterministic (no order depends on atomics).
 */
moe_status moe_group(const int32_t* topk_ids, int n_tokens, int top_k, int n_experts,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                     int32_t* dev_error, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Workspace bytes moe_ffn_forward (and its two stages) need for n_tokens. */
size_t moe_ffn_workspace_bytes(const moe_layer* layer, int n_tokens);

/*
 * A second copy of a layer's expert weights in the order the batched gate/up
 * and down (and the single-token kernel) read them: the same codes and UE8M0
 * scale bytes ("DeepSeek V4 target engine (CPU + optional CUDA tier)": MXFP4
 * routed experts, fp8-e4m3 + UE8M0 dense weights; the layout itself is this
 * library's, for this GPU's matrix instructions).  In the row-major arrays
 * a 128-input step of 16 rows touches 64 (MXFP4) or 128 (fp8) bytes of each
 * of 16 rows; packed, it is one (two) contiguous KiB, and the scale bytes of
 * four steps of a lane are one 32-bit word.
 *
 * moe_packed_experts_bytes: bytes of the copy for `layer` (the routed gate,
 *   up and down matrices and the shared expert's three), or 0 when the layer
 *   cannot be packed: routed experts not MXFP4, or hidden, inter (or
 *   shared_inter) not a multiple of 512.
 * moe_pack_experts: writes the copy into `packed` (device, 256-byte
 *   aligned, at least moe_packed_experts_bytes(layer) bytes; the caller owns
 *   it), asynchronously on `stream`, reading the layer's arrays.  Returns
 *   MOE_ERR_UNSUPPORTED for a layer that cannot be packed, MOE_ERR_INVALID
 *   for a NULL or misaligned buffer or a short size.  Set
 *   layer->packed_experts = packed afterwards to use it.  Results are
 *   bitwise equal with and without it, except for the batches of
 *   moe_ffn_forward that then take the E2M3 parts of h (see its numerics:
 *   at least 16 routed slots per expert, bf16 x, intermediate sizes up to
 *   2048), whose y stays within the same tolerance of the exact result.
 * Layout, for each matrix of R rows x C inputs (R/16 row blocks of 16 rows,
 * S = C/128 steps, lane l = 16*g + r):
 *   MXFP4 codes: block b step s at byte (b*S + s)*1024, lane l holding the
 *     16 code bytes of row 16b + r, inputs 128s + 32g .. +31;
 *   fp8 codes: block b step s half h at byte ((b*S + s)*2 + h)*1024, lane l
 *     holding row 16b + r, inputs 128s + 64h + 16g .. +15;
 *   scales (both): block b, steps 4c .. 4c+3 at byte (b*S/4 + c)*256, lane l
 *     holding in byte t the scale of row 16b + r for step 4c+t (MXFP4: of
 *     its inputs 128(4c+t) + 32g .. +31; fp8: the row's one scale of the
 *     step).
 * Matrices in the order gate, up, down, shared gate, shared up, shared down,
 * codes then scales, each section 256-byte aligned; scales take R*C/32 bytes
 * in both formats.
 */
size_t moe_packed_experts_bytes(const moe_layer* layer);
moe_status moe_pack_experts(const moe_layer* layer, void* packed, size_t packed_bytes,
                            hipStream_t stream);

/*
 * Expert FFN and combine ("Deep-Dive Mathematical & Kernel Guide", section 4
 * SwiGLU equation and section 3.2 combine equation):
 *   y[t] = e_shared(x_t) + sum_i topk_w[t][i] * e_{topk_ids[t][i]}(x_t),
 *   e(x) = W_down (SiLU(W_gate x) * (W_up x)), SiLU(g) = g / (1 + exp(-g)).
 *   x        [n_tokens][hidden], fp32 or bf16 (x_type), 16-byte aligned.
 *   topk_w   fp32 [n_tokens][top_k] as made by a router.
 *   counts, offsets, perm, inv_perm   as made by moe_group for the same ids.
 *   y        out fp32 [n_tokens][hidden], fully overwritten.
 *   The slots' experts come from counts/offsets/perm/inv_perm; the ids
 *   themselves are not read.
 * Numerics (all products accumulate in fp32 on the matrix cores):
 *   - bf16 x with more than 16 tokens, a hidden size the small-batch
 *     kernel does not cover, or an fp8 expert (routed or shared): the
 *     grouped GEMMs.  Weight codes and scale bytes go undecoded into the scaled
 *     matrix instruction; x is first rewritten as two E4M3 parts under one
 *     power-of-two scale per 32 inputs (hi + lo sum back to the bf16 value
 *     exactly for inputs within 2^-13 of their block's largest magnitude;
 *     smaller ones keep their bits above 2^-17 of that magnitude); the
 *     SwiGLU output h is stored as three E4M3 parts per 32 values (h to
 *     2^-12 of its magnitude) for the down projection.  With the packed
 *     copy (moe_pack_experts) of MXFP4 experts, batches of at least 16
 *     slots per routed expert and intermediate sizes up to 2048 store h
 *     instead as three E2M3 parts per 32 values, each part under its own
 *     power-of-two scale (h to 2^-12 of its block's largest magnitude), and
 *     the down projection multiplies them on the 32x32x64 form of the
 *     instruction.
 *   - bf16 x with MXFP4 experts and up to 16 tokens: weights decoded
 *     exactly to bf16 in registers, x as given, h as a bf16 high + low pair
 *     (16 significant bits).
 *   - fp32 x: weights decoded exactly to bf16, x and h as bf16 high + low
 *     pairs.
 *   Either way the error stays far inside max|err| <= 2e-3 * rms(y) of the
 *   exact result for inputs like the pages' workloads.  The combine sums each
 *   token's terms in a fixed order (shared first, then slot 0..top_k-1), so
 *   y is deterministic.
 */
moe_status moe_ffn_forward(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                           const float* topk_w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv_perm, float* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_ffn_forward with the gate-first lazy skip of moe_opts (lazy_tau; the
 * routing options are ignored here) and, for benchmarks, the events of
 * moe_ffn_forward_timed (each nullable).  The workspace size is
 * moe_ffn_workspace_bytes's.
 */
moe_status moe_ffn_forward_ex(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                              const float* topk_w, const int32_t* counts, const int32_t* offsets,
                              const int32_t* perm, const int32_t* inv_perm, float* y,
                              const moe_opts* opts, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t gate_up_start,
                              hipEvent_t gate_up_stop, hipEvent_t down_start,
                              hipEvent_t down_stop);

/*
 * The two stages of moe_ffn_forward, for callers that time or interleave
 * them; the same arguments, run in this order on the same workspace.
 *   moe_ffn_gate_up: gate/up matmuls with on-the-fly decode and SwiGLU,
 *                    writing h into the workspace.
 *   moe_ffn_down:    down projection, routing weights and combine into y.
 */
moe_status moe_ffn_gate_up(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                           const float* topk_w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv_perm, float* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
moe_status moe_ffn_down(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                        const float* topk_w, const int32_t* counts, const int32_t* offsets,
                        const int32_t* perm, const int32_t* inv_perm, float* y,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_ffn_forward that also records, into caller-created events (each may
 * be NULL), the start and end of the kernel that runs the routed experts'
 * gate/up and of the kernel that runs their down projection (the shared
 * expert is in the same kernel when it has the routed experts' weight type,
 * and an fp8 shared expert next to packed MXFP4 routed experts when h
 * goes to the down as E2M3 parts: at least 16 routed slots per expert,
 * intermediate sizes up to 2048, the quantized activations below 2 GiB;
 * the activation quantization of batched calls, a shared expert in
 * launches of its own and the combine pass run outside the timed pairs).
 * The times come from the kernels' own dispatches, so no extra packets are
 * queued and the stream runs as it would untimed.  For benchmarks and
 * profilers: hipEventElapsedTime(start, stop) is the kernel's duration.
 */
moe_status moe_ffn_forward_timed(const moe_layer* layer, const void* x, int x_type,
                                 int n_tokens, const float* topk_w, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* perm,
                                 const int32_t* inv_perm, float* y, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t gate_up_start, hipEvent_t gate_up_stop,
                                 hipEvent_t down_start, hipEvent_t down_stop);

/*
 * The whole layer from router logits: learned routing, grouping and the FFN
 * ("Deep-Dive Mathematical & Kernel Guide", sections 1, 3.2 and 4), with the
 * semantics of moe_route_group followed by moe_ffn_forward, in one call.
 *   logits        fp32 [n_tokens][layer->n_experts]; routed_scale > 0.
 *   topk_ids, topk_w, counts, offsets, perm, inv_perm
 *                 out, as written by moe_route_group.
 *   x, x_type, y  as for moe_ffn_forward.
 *   workspace     caller-owned device memory of at least
 *                 moe_forward_workspace_bytes(layer, n_tokens) bytes,
 *                 16-byte aligned.  Its first MOE_FORWARD_SYNC_BYTES hold a
 *                 launch counter and barrier flags stamped with it; the
 *                 single-token kernel advances the counter itself, so the
 *                 words need no reset between calls and a call captured in a
 *                 HIP graph may be replayed.  Zero them once with
 *                 moe_forward_workspace_init before the first call.  Calls
 *                 that share a workspace must not overlap in time.
 *   dev_error     nullable; MOE_DEVERR_SYNC is set if a wait of the
 *                 single-token kernel times out.
 * Single-token calls with bf16 activations, MXFP4 routed experts (and an
 * MXFP4 shared expert of the same width), n_experts <= 256, hidden in
 * {512, 1024, 2048, 4096} and inter a multiple of 128 up to 4096 run as one kernel
 * when the GPU holds at least hidden/16 of its workgroups at once (256 on
 * MI355X); every other call runs the route+group kernel and the FFN kernels
 * of moe_ffn_forward.
 * Co-residency: the single kernel's grid is the number of its workgroups the
 * occupancy query says fit on the GPU at once (one per compute unit), and
 * its workgroups meet at a grid barrier, so it needs all of them resident
 * together.  Kernels of other streams or processes that hold compute units
 * (or their LDS) for the whole call, a GPU partitioned below its full count
 * of compute units, or a debugger that serialises workgroups break that.
 * The barrier's wait is bounded (about a second of polling): a workgroup
 * that gives up sets MOE_DEVERR_SYNC in *dev_error and writes NaN into the
 * rows of y it owns, so an incomplete y never looks like a result even when
 * dev_error is NULL.
 */
#define MOE_FORWARD_SYNC_BYTES 8192
/* 1 if moe_forward runs as the single fused kernel for this layer, batch
 * size and activation type (then its grid barrier needs the whole GPU), 0 if
 * it runs the separate kernels, -1 for an invalid layer. */
int moe_forward_single_kernel(const moe_layer* layer, int n_tokens, int x_type);
size_t moe_forward_workspace_bytes(const moe_layer* layer, int n_tokens);
moe_status moe_forward_workspace_init(void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
moe_status moe_forward(const moe_layer* layer, const float* logits, float routed_scale,
                       const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                       float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, float* y, void* workspace, size_t workspace_bytes,
                       int32_t* dev_error, hipStream_t stream);
/* moe_forward with start/stop events (nullable) around the whole layer: the
 * single-token kernel records them from its own dispatch; the multi-kernel
 * path records start before its first kernel and stop after its last. */
moe_status moe_forward_timed(const moe_layer* layer, const float* logits, float routed_scale,
                             const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                             int32_t* inv_perm, float* y, void* workspace,
                             size_t workspace_bytes, int32_t* dev_error, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop);

/*
 * moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments and results as moe_forward, without the workspace: the
 * scratch memory is an array of MOE_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU it runs on, held until the process ends.  Nothing is allocated
 * by the call (the first call on a device also enqueues one small kernel that
 * clears the array's barrier flags).
 *   Batches whose moe_forward_workspace_bytes exceed
 *   MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before anything is
 *   enqueued (at hidden 4096, intermediate 2048, top-6 and a shared expert:
 *   up to about 370 tokens).
 *   Every call on a GPU uses that GPU's one array and leaves its contents
 *   behind: calls on one GPU must not overlap in time (two streams, or two
 *   host threads, running calls at once on the same device race on it).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_layer* layer, const float* logits, float routed_scale,
                               const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_perm, float* y, int32_t* dev_error,
                               hipStream_t stream);

/*
 * moe_forward with the options of moe_opts (routing options and the lazy
 * skip) and start/stop events (nullable) as moe_forward_timed.  Single-token
 * calls with group-limited selection, a selection bias or tail pruning still
 * run as the one fused kernel (same conditions as moe_forward); a lazy skip
 * runs the separate kernels, whose small-batch gate/up then goes gate first.
 */
moe_status moe_forward_ex(const moe_layer* layer, const float* logits, float routed_scale,
                          const moe_opts* opts, const void* x, int x_type, int n_tokens,
                          int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv_perm, float* y, void* workspace,
                          size_t workspace_bytes, int32_t* dev_error, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop);

/* A static, human-readable name of a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
