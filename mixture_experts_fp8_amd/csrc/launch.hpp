// Internal launchers of the A8W4 MoE kernels (host side).  Arguments are
// validated by the C ABI in api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct GemmArgs {
  int32_t M;              // tokens
  int32_t topk;
  int32_t N;              // rows of the expert weight matrix (2I for stage 1, H for stage 2)
  int32_t K;              // reduction length (H for stage 1, I for stage 2)
  int32_t bm;             // rows per sorted block
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  const uint8_t* bq;      // B rows: token activations (stage 1) or sorted intermediate (stage 2), [.., K]
  const uint8_t* bs;      // their E8M0 scales [.., K/32]
  const uint8_t* w;       // packed expert weights, N*K/2 bytes per expert
  const uint8_t* ws;      // packed scales, N*K/32 bytes per expert
  uint8_t* out_q;         // stage 1: intermediate codes [P, N/2]
  uint8_t* out_s;         // stage 1: intermediate scales [P, N/64]
  const float* topk_weights;  // stage 2: [M, topk]
  int16_t* y_codes;       // stage 2: weighted route outputs [M, topk, N], 16-bit codes
  uint8_t* y_exps;        //          and their exponent bytes [M, topk, N/32]
};

// Cross-workgroup state of the fused decode launch (stage one, stage two and
// the top-k combine in one kernel).  The counters are zero on entry and the
// launch leaves them zero; status stays 0 unless a wait gave up.
constexpr int kCounterStride = 64;   // int32 per block_done entry (one 256-byte run each)

struct FusedArgs {
  int32_t* block_done;    // [blocks * kCounterStride] stage-one tiles finished, per sorted block
  int32_t* block_seen;    // [blocks] stage-two tiles past their wait, per block
  int32_t* token_done;    // [M, stage-two tiles per block] routes finished per token and column range
  int32_t* status;        // [1]
  const int32_t* topk_ids;  // [M, topk] global expert ids
  int32_t num_experts;    // E held here
  int32_t expert_offset;  // global id of local expert 0
  uint16_t* out;          // [M, H] BF16 output
  int32_t ng1;            // stage-one tiles per block (set by the launcher)
  int32_t g1, g2;         // workgroups of the stage-one and stage-two regions (set by the launcher)
};

// Router inputs and outputs (softmax top-k of the logits, optional shared slot).
struct RouteArgs {
  const float* logits;    // [M, routed] router logits; null: the ids are given
  int32_t routed;         // logits per token
  int32_t k_routed;       // routed slots per token
  int32_t shared;         // expert id of the extra shared slot, or -1
  int32_t* ids;           // [M, k_routed + (shared >= 0)] out
  float* weights;         // same shape, out
};

// One launch: the first workgroups sort the routes (skipped if ids is null),
// the others quantise x [M, H] (skipped if x is null).  With ra.logits set the
// routes come from the router (ids = ra.ids): inside the sort workgroup when
// a single one sorts, else in a launch of its own before.
hipError_t launch_prep(const int32_t* ids, int32_t M, int32_t topk, int32_t E, int32_t expert_offset,
                       int32_t bm, int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                       const uint16_t* x, int64_t H, uint8_t* q, uint8_t* s, const RouteArgs& ra,
                       hipStream_t stream);
hipError_t launch_route(const RouteArgs& ra, int32_t M, hipStream_t stream);
hipError_t launch_combine(int64_t M, int32_t H, int32_t topk, int32_t E, int32_t expert_offset,
                          const int32_t* ids, const int16_t* y_codes, const uint8_t* y_exps,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_pack(const uint8_t* src, const uint8_t* src_s, uint8_t* dst, uint8_t* dst_s,
                       int64_t E, int64_t N, int64_t K, hipStream_t stream);
// max_blocks: upper bound of sorted blocks (grid size); kernels read the real count on device
hipError_t launch_stage1(const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
hipError_t launch_stage2(const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
// Stage one (a1), stage two (a2) and the combine in one launch, bm = 16 or 32
// (gemm.hip); the counters of fa must be zero
hipError_t launch_fused(const GemmArgs& a1, const GemmArgs& a2, const FusedArgs& fa, int64_t max_blocks,
                        hipStream_t stream);
// A16W4 variant (gemm_a16.hip), bm = 16 or 32: stage one writes a BF16
// intermediate [capacity, I] to a.out_q from BF16 rows a.bq; stage two reads it
hipError_t launch_a16_stage1(const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
hipError_t launch_a16_stage2(const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
// its LDS-tiled form for bm = 64 or 128 (gemm_tile.hip)
hipError_t launch_a16_tile(int stage, const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
// LDS-tiled variant of either stage for bm = 64 or 128 (gemm_tile.hip)
hipError_t launch_tile(int stage, const GemmArgs& a, int64_t max_blocks, hipStream_t stream);
// n independent 16 x 16 scaled MFMAs, A scale as byte sel of its operand (probe.hip)
hipError_t launch_mfma_probe(int64_t n, int sel, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, float* d, hipStream_t stream);
// weight streaming in the decode stage-one shape, packed (layout 0) or raw
// row-major (1) MXFP4 weights of groups * 64 rows x K (probe.hip)
hipError_t launch_stream_probe(int layout, int64_t groups, int K, const uint8_t* w, const uint8_t* ws,
                               uint32_t* out, hipStream_t stream);
// n independent 16 x 16 x 32 BF16 MFMAs (probe.hip)
hipError_t launch_mfma_bf16_probe(int64_t n, const uint16_t* a, const uint16_t* b, float* d,
                                  hipStream_t stream);

}  // namespace moe
