/*
 * moe_a8w4.h -- C ABI of the A8W4 fused mixture-of-experts layer for MI355X
 * (gfx950): FP8 E4M3 activations with per-1x32 E8M0 scales times MXFP4
 * (E2M1 + E8M0 per 1x32) expert weights, BF16 output.
 *
 * One call computes the layer defined in aiter PR 5609 ("Add DeepSeek V4.1
 * Flash TP4 gfx950 MoE tuning", section Configuration) -- 8-bit float
 * activations against 4-bit MX expert weights with a power-of-two scale per
 * 32 elements, gate and up rows alternating in one matrix, a SiLU gate, the
 * routing probability applied after the down projection, a bfloat16
 * result -- and spans what the timed call of aiter PR 5904 ("Add tuned a8w4
 * fused-MoE configs for DeepSeek V4.1-Flash (TP4 + EP, gfx950)", section
 * "Fused-MoE kernel, expert-parallel benchmark") spans: grouping the routes
 * by expert, both GEMMs and the re-quantisation between them.
 *
 *   a_q, a_s  = per-1x32 quantisation of hidden (E8M0 exponent
 *               floor(log2 amax) - 8, clamped at -127; E4M3 elements rounded
 *               to nearest even, saturating at 448)
 *   for every route (t, k) whose expert g = topk_ids[t,k] is local,
 *   e = g - expert_offset in [0, E):
 *     gate_j = <a_t, w13[e, 2j]>, up_j = <a_t, w13[e, 2j+1]>   (j < I)
 *     h      = per-1x32 quantisation of SiLU(gate) * up
 *     y      = w2[e] h                                          (H values)
 *   out[t] = BF16( sum over local k of topk_weights[t,k] * y_(t,k) )
 *   Routes of non-local experts contribute nothing; a token with none gets 0.
 *   Each term is formed in float32 and held in the route-row format of
 *   moe_a8w4_stage2 (error at most 2^-14 of the largest magnitude of its
 *   32-output block) before the float32 sum in ascending k.
 *
 * Conventions
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and never synchronises:
 *     every entry point only enqueues work on `stream` and returns.  Buffers
 *     must stay alive until that work completes.  Inputs are never written.
 *   - Return value: 0 on success; a negative MOE_ERR_* if the arguments are
 *     invalid, in which case nothing was enqueued; a positive hipError_t if a
 *     launch failed.  Faults inside kernels surface at the caller's next
 *     synchronisation.  moe_a8w4_status_str() names a code.
 *   - Every pointer must be 16-byte aligned (the workspace 256-byte aligned).
 *   - Limits: 0 <= M < 2^24; H a positive multiple of 512; I a positive
 *     multiple of 128; 1 <= E <= 512; 1 <= topk <= 8.
 *   - No data-dependent value is read back to the host, so calls can be
 *     captured in a HIP graph and replayed on changed inputs.
 */
#ifndef MOE_A8W4_H
#define MOE_A8W4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL */
#define MOE_ERR_DIMS (-2)      /* a dimension is outside the limits above */
#define MOE_ERR_ALIGN (-3)     /* a pointer is not 16-byte (workspace: 256-byte) aligned */
#define MOE_ERR_WORKSPACE (-4) /* workspace_bytes smaller than moe_a8w4_workspace_bytes() */
#define MOE_ERR_BLOCK_M (-5)   /* block_m not one of 16, 32, 64, 128 */
#define MOE_ERR_SCRATCH (-6)   /* moe_a8w4_forward_noalloc: the call needs more than
                                  MOE_A8W4_NOALLOC_SCRATCH_BYTES of workspace */

/* Size of the static device scratch of moe_a8w4_forward_noalloc (per GPU). */
#define MOE_A8W4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef struct moe_a8w4_dims {
  int32_t tokens;        /* M: token rows in hidden / out / topk_* */
  int32_t hidden;        /* H: model width */
  int32_t inter;         /* I: intermediate width as stored (zero-padded columns included) */
  int32_t num_experts;   /* E: experts held in the weight tensors */
  int32_t expert_offset; /* global id of weight expert 0 (a rank's local-expert slice) */
  int32_t topk;          /* slots per token */
  int32_t routed_experts;/* experts the router chooses among, if more than num_experts
                            (a local slice); 0 = num_experts.  Only sizes the blocks. */
} moe_a8w4_dims;

/* ------------------------------------------------------------------ sizes */

/* Bytes of workspace moe_a8w4_forward needs for these dims (an upper bound
 * independent of the routing): the values one call passes between its steps
 * -- quantised activations, the sort, the re-quantised intermediate, the
 * weighted route rows (aiter PR 5904, "Fused-MoE kernel, expert-parallel
 * benchmark": one call spans sorting, both GEMMs and the re-quantisation
 * between them).  Writes *bytes; returns a status. */
int moe_a8w4_workspace_bytes(const moe_a8w4_dims* dims, size_t* bytes);

/* Rows per sorted block (16, 32, 64 or 128) that moe_a8w4_forward uses for
 * these dims: a function of the mean routes per expert,
 * M * topk / max(num_experts, routed_experts), only.  Negative status if
 * invalid.  The same block_m is shared by the sort and both stages (aiter
 * PR 5609, Commands run: the sort's block must equal the stage-two tile). */
int moe_a8w4_block_m(const moe_a8w4_dims* dims);

/* Capacity, in entries, that sorted_ids needs for these dims and block_m
 * (every expert's run padded to a multiple of block_m, as the sort emits it):
 * R + min(E, R) * (block_m - 1) rounded up to block_m, R = M * topk.
 * block_expert needs capacity / block_m entries.  Negative status if invalid. */
int64_t moe_a8w4_sort_capacity(const moe_a8w4_dims* dims, int32_t block_m);

/* ---------------------------------------------------------------- weights */

/* Reorder MXFP4 expert weights into the layout the GEMM kernels stream
 * (a one-time, off-path transform, part of this interface: moe_a8w4_forward
 * and the step entry points take its outputs; the packed buffers have the
 * same sizes as the inputs).  The weights are those of aiter PR 5609,
 * "Add DeepSeek V4.1 Flash TP4 gfx950 MoE tuning", Configuration (MXFP4 with
 * one E8M0 scale per 32 along K, gate and up rows interleaved).  Packing is a
 * permutation of bytes, so the layer computes exactly what it would on the
 * raw layout; reading the raw layout in the order the matrix instruction
 * wants instead streams at 3.1 TB/s against 6.8 TB/s (measured in the decode
 * stage-one shape: moe_a8w4_stream_probe).  Inputs, row-major, element 2i in
 * the low nibble of byte i:
 *   w13      [E, 2I, H/2]  E2M1 codes; row 2j = gate of column j, row 2j+1 = up
 *   w13_s    [E, 2I, H/32] E8M0 scale of each run of 32 elements along H
 *   w2       [E, H, I/2]   E2M1 codes
 *   w2_s     [E, H, I/32]  E8M0 scales along I
 * Outputs: w13_p, w13_s_p, w2_p, w2_s_p of the same byte sizes. */
int moe_a8w4_pack_weights(const moe_a8w4_dims* dims, const uint8_t* w13, const uint8_t* w13_s,
                          const uint8_t* w2, const uint8_t* w2_s, uint8_t* w13_p, uint8_t* w13_s_p,
                          uint8_t* w2_p, uint8_t* w2_s_p, hipStream_t stream);

/* ------------------------------------------------------------ the router */

/* Router of the backbone configurations (the workloads' "softmax top-k of the
 * router logits, renormalised"; the prefill configuration's fused shared
 * expert): for each token, the k_routed largest of its routed_experts logits
 * in descending order (equal values: the lower expert id first), weighted by
 * the softmax of the chosen logits -- the softmax over all routed_experts
 * renormalised over the chosen ones, which is the same in exact arithmetic;
 * computed in float32 (the ids are exact, the weights within a few ulp).
 * With shared_expert >= 0 a last slot holds that expert id with weight 1.
 *   logits        [M, routed_experts] float32
 *   topk_ids      [M, k] int32 out, k = k_routed + (shared_expert >= 0)
 *   topk_weights  [M, k] float32 out
 * Limits: 1 <= k_routed <= routed_experts <= 512, k <= 8. */
int moe_a8w4_route(int32_t M, int32_t routed_experts, int32_t k_routed, int32_t shared_expert,
                   const float* logits, int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* ------------------------------------------------------------- the layer */

/* The whole layer: quantise, sort, stage one, stage two, BF16 output, as
 * four launches (quantiser with the sort, stage one, stage two, combine). 
 *   hidden        [M, H] BF16
 *   topk_ids      [M, topk] int32 global expert ids (any value; non-local skipped)
 *   topk_weights  [M, topk] float32
 *   w13_p, w13_s_p, w2_p, w2_s_p   weights packed by moe_a8w4_pack_weights
 *   out           [M, H] BF16, every element overwritten
 *   workspace     >= moe_a8w4_workspace_bytes(dims) bytes, contents ignored
 * M = 0 enqueues nothing and succeeds. */
int moe_a8w4_forward(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                     const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                     const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * moe_a8w4_forward with no workspace argument.  Its workspace is a static
 * array of MOE_A8W4_NOALLOC_SCRATCH_BYTES (64 MiB) in device memory, one per
 * GPU the library runs on, held until the process ends; the call allocates
 * nothing (its first call on a device looks up that device's array).  Calls
 * whose moe_a8w4_workspace_bytes() exceeds that size return MOE_ERR_SCRATCH
 * and enqueue nothing (64 MiB covers, e.g., 384 experts top-6 at I 640 up to
 * 768 tokens).  Every call on a GPU shares its array: calls that overlap on
 * one GPU (other streams, other host threads) race and give undefined
 * results; calls on one stream are ordered and safe.  Other arguments,
 * results and errors as moe_a8w4_forward. */
int moe_a8w4_forward_noalloc(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                             const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, hipStream_t stream);

/* The whole layer from the router logits: moe_a8w4_route (with
 * routed_experts = dims->routed_experts, k_routed = dims->topk minus the
 * shared slot), writing topk_ids / topk_weights [M, dims->topk] (caller-owned
 * outputs, left holding the routing), then moe_a8w4_forward on them.  When
 * one workgroup sorts and M <= 16, the routing runs inside the sort's launch
 * (no launch of its own).  Other arguments as moe_a8w4_forward. */
int moe_a8w4_forward_routed(const moe_a8w4_dims* dims, const void* hidden, const float* router_logits,
                            int32_t shared_expert, int32_t* topk_ids, float* topk_weights,
                            const uint8_t* w13_p, const uint8_t* w13_s_p, const uint8_t* w2_p,
                            const uint8_t* w2_s_p, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ----------------------------------------------- the steps, one at a time */

/* Per-1x32 FP8 quantisation of BF16 rows (the activation quantisation of
 * aiter PR 5609, Configuration: FP8 activations, per-1x32 scaling; OCP MX
 * v1.0 conversion): x [M, H] -> q [M, H] E4M3 codes, s [M, H/32] E8M0 codes.
 * H must be a multiple of 32; every pointer 16-byte aligned. */
int moe_a8w4_quant_act(int32_t M, int32_t H, const void* x, uint8_t* q, uint8_t* s,
                       hipStream_t stream);

/* The sorting step of one call (aiter PR 5904, "Fused-MoE kernel,
 * expert-parallel benchmark": sorting is part of the timed call; aiter PR
 * 5609, Commands run: its block size matches the stage-two tile).
 * Group local routes by expert: sorted_ids [capacity] receives, expert by
 * expert in ascending local id, the expert's routes in ascending t*topk + k
 * as (k << 24) | t, each expert's run padded with M to a multiple of block_m
 * (experts without routes get no rows); block_expert [capacity/block_m]
 * receives the local expert of each block; num_padded [1] the total rows.
 * Entries past num_padded are left unspecified.  The result does not
 * depend on timing (bitwise repeatable).  Every pointer 16-byte aligned
 * (topk_ids is read 16 bytes at a time), else MOE_ERR_ALIGN. */
int moe_a8w4_sort(const moe_a8w4_dims* dims, int32_t block_m, const int32_t* topk_ids,
                  int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                  hipStream_t stream);

/* moe_a8w4_quant_act and moe_a8w4_sort of one call in a single launch (the
 * sort's workgroups, one per 1024 routes up to 64, run beside the
 * quantiser's): the first step of moe_a8w4_forward.  Same buffers and
 * contracts as the two calls. */
int moe_a8w4_quant_sort(const moe_a8w4_dims* dims, int32_t block_m, const void* hidden,
                        const int32_t* topk_ids, uint8_t* a_q, uint8_t* a_s, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_padded, hipStream_t stream);

/* Stage one of aiter PR 5609, Configuration (gate/up GEMM on interleaved
 * rows, SiLU(gate) * up, no routing weight) with the intermediate
 * quantisation of aiter PR 5904, "Fused-MoE kernel, expert-parallel
 * benchmark", for every sorted block: inter_q [capacity, I] E4M3 codes and
 * inter_s [capacity, I/32] E8M0 codes, row p = sorted position, holding the
 * per-1x32 quantisation of SiLU(gate) * up.  Rows of blocks that hold a
 * route are written in full (padding columns included); rows past the last
 * route of a block may be left unwritten. */
int moe_a8w4_stage1(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* a_q,
                    const uint8_t* a_s, const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const uint8_t* w13_p, const uint8_t* w13_s_p,
                    uint8_t* inter_q, uint8_t* inter_s, hipStream_t stream);

/* Stage two of aiter PR 5609, Configuration (down projection; the routing
 * weight applied here, not in stage one): for every local route (t, k), row
 * (t, k) of y_routes receives
 * topk_weights[t,k] * (w2[e] h), h its dequantised intermediate, in the
 * route-row format: y_routes holds [M, topk, H] int16 codes followed by
 * [M, topk, H/32] uint8 exponents, M*topk*(2H + H/32) bytes in all (16-byte
 * aligned).  Each 32 consecutive outputs v of a row share an exponent S =
 * max(fp32 exponent field of their largest |v|, 14) and are stored as
 * code = round-to-nearest-even(v * 2^(140 - S)), |code| <= 2^14, read back
 * exactly as code * 2^(S - 140): an error of at most 2^-14 of the block's
 * largest magnitude, far finer than a BF16 rounding of each route's share.
 * Rows of non-local slots are not written. */
int moe_a8w4_stage2(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* inter_q,
                    const uint8_t* inter_s, const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const float* topk_weights, const uint8_t* w2_p,
                    const uint8_t* w2_s_p, void* y_routes, hipStream_t stream);

/* Top-k combine into the BF16 output of aiter PR 5609, Configuration:
 * out[t, :] (BF16, [M, H]) = round-to-nearest-even of the
 * float32 sum, in ascending k, of the decoded rows (t, k, :) of y_routes (the
 * stage-two route rows) over the token's local slots (topk_ids decides which
 * slots are local); zero for a token without one.  Bitwise repeatable. */
int moe_a8w4_combine(const moe_a8w4_dims* dims, const int32_t* topk_ids, const void* y_routes,
                     void* out, hipStream_t stream);

/* Stage one, stage two and the top-k combine of one call in a single launch
 * (block_m 16 or 32), the decode form of the layer after moe_a8w4_quant_sort
 * (aiter PR 5904, "Fused-MoE kernel, expert-parallel benchmark": the timed
 * call spans the grouping, both GEMMs and the re-quantisation).  Results as
 * moe_a8w4_stage1 (inter_q, inter_s), moe_a8w4_stage2 (y_routes) and
 * moe_a8w4_combine (out, every element written) with the same buffers.
 * A stage-two tile of a block starts streaming its weights at once and waits
 * for that block's stage-one tiles through counters in device memory; the
 * workgroup that finishes a token's last route over a range of output
 * columns sums that range.
 *   counters  int32 [moe_a8w4_fused_counters(dims, block_m)], caller-owned:
 *             must hold zeros on entry; a completed call leaves them zero.
 *             counters[0] is a status word: nonzero if a wait gave up after
 *             about 0.5 s (only possible when the GPU cannot run all of the
 *             launch's earlier workgroups, e.g. it is shared), in which case
 *             the outputs and counters are invalid.
 * Calls sharing a counters buffer must not overlap.  Entries past
 * num_padded of the sort buffers are ignored. */
int moe_a8w4_stages_fused(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* a_q,
                          const uint8_t* a_s, const int32_t* sorted_ids, const int32_t* block_expert,
                          const int32_t* num_padded, const int32_t* topk_ids, const float* topk_weights,
                          const uint8_t* w13_p, const uint8_t* w13_s_p, const uint8_t* w2_p,
                          const uint8_t* w2_s_p, uint8_t* inter_q, uint8_t* inter_s, void* y_routes,
                          int32_t* counters, void* out, hipStream_t stream);

/* Number of int32 counters moe_a8w4_stages_fused needs (negative status on
 * invalid dims, or block_m other than 16 and 32). */
int64_t moe_a8w4_fused_counters(const moe_a8w4_dims* dims, int32_t block_m);

/* ------------------------------------------------------ the A16W4 variant */

/* The A16W4 variant of the layer (aiter PR 6286, "Retune gfx942 a16w4 DSv4.1
 * tiles for Triton 3.8": w1 with the SwiGLU fused, w2 separate, BF16
 * activations, MXFP4 weights).  The same dims, weights packed by
 * moe_a8w4_pack_weights and routing as moe_a8w4_forward; the activations
 * are not quantised: stage one multiplies the BF16 hidden rows by the
 * dequantised w13 (FP32 accumulation), the intermediate SiLU(gate) * up is
 * rounded to BF16 (nearest, ties to even), stage two multiplies it by w2,
 * and the routing-weighted routes are combined as in moe_a8w4_forward.
 * Blocks of 16, 32, 64 or 128 routes (moe_a16w4_block_m); the weights are exact in
 * BF16 for every scale code whose products stay normal (codes 1 ... 254
 * with |element| >= 0.5 scaled above 2^-126).  Four launches: sort, stage
 * one, stage two, combine.  Errors, ownership and stream rules as
 * moe_a8w4_forward. */
int moe_a16w4_forward(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                      const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                      const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace moe_a16w4_forward needs for these dims. */
int moe_a16w4_workspace_bytes(const moe_a8w4_dims* dims, size_t* bytes);

/* Rows per sorted block (16, 32, 64 or 128) that moe_a16w4_forward uses. */
int moe_a16w4_block_m(const moe_a8w4_dims* dims);

/* Stage one of the A16W4 variant for every sorted block (sort buffers from
 * moe_a8w4_sort with this block_m, 16, 32, 64 or 128): inter_bf16 [capacity, I] BF16,
 * row p = sorted position, holding BF16(SiLU(gate) * up); rows of blocks
 * that hold a route are written in full. */
int moe_a16w4_stage1(const moe_a8w4_dims* dims, int32_t block_m, const void* hidden,
                     const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                     const uint8_t* w13_p, const uint8_t* w13_s_p, void* inter_bf16, hipStream_t stream);

/* ------------------------------------------------------ hardware probe */

/* The scaled matrix instruction both GEMMs are built from
 * (v_mfma_scale_f32_16x16x128_f8f6f4 with an MXFP4 A and an FP8 B operand),
 * once per 16 x 16 tile, from a zero accumulator; exported so that its
 * operand layout, scale-byte selection and accumulation error can be
 * measured against exact arithmetic (the local error budget of the
 * requantised intermediate rests on that error).  For tile i < n:
 *   a_fp4   [n, 16, 64]   E2M1 codes of rows m, K = 128 (element 2c low nibble)
 *   a_scale [n, 16, 4]    E8M0 scale of row m's K block of 32
 *   b_fp8   [n, 16, 128]  E4M3 codes of columns c
 *   b_scale [n, 16, 4]    E8M0 scale of column c's K block of 32
 *   d       [n, 16, 16]   float32 out: sum over K of the scaled products
 * byte_sel (0..3) is the byte of its 32-bit operand that carries A's scale
 * (the other bytes hold an invalid code).  Limits: 0 <= n <= 2^24. */
int moe_a8w4_mfma_probe(int64_t n, int32_t byte_sel, const uint8_t* a_fp4, const uint8_t* a_scale,
                        const uint8_t* b_fp8, const uint8_t* b_scale, float* d, hipStream_t stream);

/* The BF16 matrix instruction of the A16W4 variant (v_mfma_f32_16x16x32_bf16),
 * once per 16 x 16 tile from a zero accumulator, for the same kind of
 * measurement: a_bf16 [n, 16, 32] rows, b_bf16 [n, 16, 32] columns (BF16
 * bits), d [n, 16, 16] float32 out = sum over K of the products.  Every
 * pointer 16-byte aligned; 0 <= n <= 2^24. */
int moe_a16w4_mfma_probe(int64_t n, const void* a_bf16, const void* b_bf16, float* d, hipStream_t stream);

/* Weight streaming in the shape of the decode stage-one kernel, for the
 * measurement behind the packed layout of moe_a8w4_pack_weights: one
 * workgroup per 64-row group of `rows` rows of K, 4 waves splitting K, every
 * lane loading one MFMA tile's A operand per K step with non-temporal 16-byte
 * loads, from the packed layout (layout 0: w, w_s as moe_a8w4_pack_weights
 * writes them for rows x K) or from the raw row-major one (layout 1: w
 * [rows, K/2], w_s [rows, K/32]).  out [rows / 64 * 4] uint32 receives one
 * fold of the loaded bytes per wave; raw weights and their packed form give
 * the same words.  rows a multiple of 64, K of 512; 16-byte aligned
 * pointers. */
int moe_a8w4_stream_probe(int32_t layout, int64_t rows, int32_t K, const uint8_t* w, const uint8_t* w_s,
                          uint32_t* out, hipStream_t stream);

/* Name of a status code (static string). */
const char* moe_a8w4_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_A8W4_H */
