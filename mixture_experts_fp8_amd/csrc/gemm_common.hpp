// Pieces shared by the two grouped-GEMM kernels of the A8W4 MoE layer
// (gemm.hip for decode-sized blocks, gemm_tile.hip for larger ones): the
// scaled MFMA, the XCD-aware tile order and the two epilogues.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

// v_mfma_scale_f32_16x16x128_f8f6f4 with A = FP4 weights (format 4) and B = FP8
// tokens (format 0).  Operand layout (measured on gfx950): A lane l holds row
// l%16, K [32(l/16), +32) in 16 bytes, low nibble first; B lane l holds column
// l%16, K [16(l/16), +16) in bytes 0..15 and K [64 + 16(l/16), +16) in bytes
// 16..31; the scale operand of lane l applies to K block l/16; the result lane
// l holds column l%16, rows 4(l/16) .. 4(l/16)+3.  OPSEL picks the scale byte.
template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_fp8(const v4i& a, const v8i& b, const v4f& c, uint32_t sa,
                                            uint32_t sb) {
  const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, OPSEL, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ v8i join8(const v4i& lo, const v4i& hi) {
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Workgroup 8j + x runs on XCD x; XCD x takes a contiguous run of the T tiles
// so that neighbouring tiles (the blocks of one expert) share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int wg, int T) {
  const int x = wg & 7, j = wg >> 3;
  const int q8 = T >> 3, rem = T & 7;
  return x * q8 + (x < rem ? x : rem) + j;
}

// Stage-one epilogue for one 64-row group and one 16-token column group of a
// wave: lane (t16, g) holds, in acc[t], rows 16g + 4t + r of the group, i.e.
// gate (r even) and up (r odd) of intermediate columns 32 grp + 8g + 2t + r/2.
// h = SiLU(gate) * up; the group's 32 columns form one per-1x32 quantisation
// block, spread over the four lanes with equal t16.  Writes row p of the
// intermediate (8 codes per lane, the scale from lane g = 0).  All 64 lanes
// must call it together.  COH: another workgroup of the launch reads it.
template <bool COH = false>
__device__ __forceinline__ void stage1_store(const v4f acc[4], int64_t p, int grp, int I, int g,
                                             uint8_t* __restrict__ out_q, uint8_t* __restrict__ out_s) {
  float h[8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float gate = acc[t][2 * q], up = acc[t][2 * q + 1];
      // SiLU with the hardware reciprocal (about 1 ulp): the result is
      // rounded to 3 mantissa bits right after
      h[2 * t + q] = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up;
    }
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(h[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const int E = block_exponent(amax);
  const uint2 q = encode8(h, exp2_neg(E));
  st64<COH>(out_q + p * I + grp * 32 + 8 * g, (uint64_t)q.x | ((uint64_t)q.y << 32));
  if (g == 0) st8<COH>(out_s + p * (I / 32) + grp, (uint8_t)(E + 127));
}

// Route slot t * topk + k of a sorted id.
__device__ __forceinline__ int64_t route_slot(int rid, int topk) {
  return (int64_t)(rid & 0xFFFFFF) * topk + (rid >> kSentinelShift);
}

// Orders one wave's LDS writes before its following LDS reads (and the
// reverse): the lanes of a wave run in lockstep, the fences make the compiler
// keep the order and wait for the outstanding LDS operations.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bytes of wave-private LDS scratch stage2_store needs: 16 rows of 128 B,
// padded to 144 so that the 16 rows start in distinct bank groups.
constexpr int kStage2Scratch = 16 * 144;

// Stage-two epilogue for one 64-row group and one 16-route column group of a
// wave: lane (t16, g) holds output columns 64 grp + 16g + 4t + r of the route
// in slot `slot` (negative: no route), wt its routing weight.  The values
// wt * acc go to that route's row in the route-row format (16-bit codes, one
// exponent byte per 32 columns; the group holds two such blocks, columns
// 0..31 in lanes g = 0, 1 and 32..63 in g = 2, 3).  The codes go through the
// wave's LDS scratch so that each store instruction writes 8 routes x 128 B
// in a row instead of 32-byte pieces of 16 routes.  All 64 lanes must call it
// together.  COH: another workgroup of the launch reads the rows.
// The slots written by store q (q = 0, 1) of stage2_store in this lane: lane
// l writes route 8 q + l / 8 of the column group, whose slot lane (route, g)
// holds (negative: none).  Route slots stay below 2^27 (tokens below 2^24,
// top-k at most 8), so 32 bits carry them.  A wave that stores several
// slices of the same routes computes them once.
__device__ __forceinline__ void stage2_store_slots(int64_t slot, int sl2[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 2; ++q) sl2[q] = __shfl((int)slot, 8 * q + (lane >> 3));
}

template <bool COH = false>
__device__ __forceinline__ void stage2_store(const v4f acc[4], int64_t slot, const int sl2[2], float wt,
                                             const GemmArgs& args, int grp, int g, uint8_t* scr) {
  const int lane = threadIdx.x & 63, t16 = lane & 15;
  // the block maximum of |wt acc|: rounding is monotonic, so |wt| times the
  // largest |acc| rounds to the largest rounded product
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(acc[t][r]));
  amax = fabsf(wt) * amax;
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  const int S = route_block_exp(amax);
  const float wm = wt * route_encode_mul(S);   // exact: a power-of-two scaling
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i0 = 2 * j, i1 = 2 * j + 1;
    w[j] = __builtin_amdgcn_perm(route_code_bits(acc[i1 >> 2][i1 & 3], wm), route_code_bits(acc[i0 >> 2][i0 & 3], wm),
                                 0x05040100u);
  }
  uint8_t* row = scr + t16 * 144 + g * 32;
  *reinterpret_cast<v4i*>(row) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  *reinterpret_cast<v4i*>(row + 16) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
  const int S1 = __shfl(S, t16 + 32);   // exponent of the second block (lane g = 2)
  wave_lds_sync();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int route = 8 * q + (lane >> 3), chunk = lane & 7;
    const v4i c = *reinterpret_cast<const v4i*>(scr + route * 144 + chunk * 16);
    if (sl2[q] >= 0) st128<COH>(args.y_codes + (int64_t)sl2[q] * args.N + grp * 64 + chunk * 8, c);
  }
  if (g == 0 && slot >= 0) st16<COH>(args.y_exps + slot * (args.N / 32) + 2 * grp, (uint16_t)(S | (S1 << 8)));
  wave_lds_sync();
}

template <bool COH = false>
__device__ __forceinline__ void stage2_store(const v4f acc[4], int64_t slot, float wt, const GemmArgs& args,
                                             int grp, int g, uint8_t* scr) {
  int sl2[2];
  stage2_store_slots(slot, sl2);
  stage2_store<COH>(acc, slot, sl2, wt, args, grp, g, scr);
}

// ------------------------------------------------ A16W4 variant pieces
//
// BF16 activations x MXFP4 weights (gemm_a16.hip, and the tile kernel in
// gemm_tile.hip): the FP4 weights are converted to BF16 in registers for the
// BF16 MFMA, and stage one rounds its SiLU(gate) * up to a BF16 intermediate.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 2^(code - 127) as an fp32 (code 0: the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  return __uint_as_float(code ? code << 23 : 0x00400000u);
}

// 8 FP4 codes (one 32-bit word, element 0 in the low nibble) to 8 BF16 times
// the scale
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  v4i r;
  r.x = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// Stage-one epilogue of the A16W4 variant: as stage1_store, but the
// intermediate is the BF16 (nearest, ties to even) of SiLU(gate) * up; lane
// (t16, g) writes the 8 consecutive columns 32 grp + 8 g .. + 7 of row p.
__device__ __forceinline__ void a16_stage1_store(const v4f acc[4], int64_t p, int grp, int I, int g,
                                                 uint16_t* __restrict__ inter) {
  uint32_t hb[8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float gate = acc[t][2 * q], up = acc[t][2 * q + 1];
      hb[2 * t + q] = f32_to_bf16(gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up);
    }
  const v4i v = {(int)(hb[0] | (hb[1] << 16)), (int)(hb[2] | (hb[3] << 16)), (int)(hb[4] | (hb[5] << 16)),
                 (int)(hb[6] | (hb[7] << 16))};
  *reinterpret_cast<v4i*>(inter + p * I + grp * 32 + 8 * g) = v;
}

}  // namespace moe
