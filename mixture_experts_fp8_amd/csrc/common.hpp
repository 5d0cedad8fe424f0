// Device-side building blocks shared by the kernels of the A8W4 MoE library:
// vector types, the FP8 E4M3 / E8M0 / BF16 conversions and the packed weight
// geometry.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;   // sort keeps per-expert state in LDS
constexpr int kMaxTopk = 8;
constexpr int kSentinelShift = 24; // sorted id = (slot << 24) | token

// ----------------------------------------------------------------- formats
//
// FP8 is OCP E4M3FN (bias 7, largest finite 448, S.1111.111 = NaN).  The block
// scale is an OCP MX E8M0 exponent; a block of 32 values with largest
// magnitude amax gets exponent E = floor(log2 amax) - 8 (8 = largest E4M3
// exponent), clamped below at -127, and elements v * 2^-E are rounded to the
// nearest E4M3 value with ties to even, saturating at 448.

// Block exponent E from the block's largest magnitude (an fp32 value).
__device__ __forceinline__ int block_exponent(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int E = ef - 127 - 8;
  return E < -127 ? -127 : E;
}

// 2^-E as an fp32 (E in [-127, 120]).
__device__ __forceinline__ float exp2_neg(int E) {
  return __uint_as_float((uint32_t)(127 - E) << 23);
}

// Route rows (stage two's per-route outputs, summed by the top-k combine).
// Each 32 consecutive outputs of a route share an exponent byte S: the fp32
// exponent field of their largest magnitude, at least 14.  Output v is stored
// as the 16-bit integer RNE(v * 2^(140 - S)), which lies in [-2^14, 2^14],
// and decodes exactly to code * 2^(S - 140); the rounding error is at most
// 2^-14 of the block's largest magnitude (blocks below 2^-112 keep 2^-127
// absolute).  Finite values only.
__device__ __forceinline__ int route_block_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return ef < 14 ? 14 : ef;
}

// 2^(140 - S) and 2^(S - 140) as fp32 (S in [14, 254]).
__device__ __forceinline__ float route_encode_mul(int S) { return __uint_as_float((uint32_t)(267 - S) << 23); }
__device__ __forceinline__ float route_decode_mul(int S) { return __uint_as_float((uint32_t)(S - 13) << 23); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> BF16 bits, nearest with ties to even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four scaled values to four E4M3 codes (element 0 lowest) with the gfx950
// conversion instruction.  With the clamp to +-448 in front, its result is the
// rule above (nearest, ties to even, saturating at 448, sign kept, subnormal
// grid of 2^-9): compared on the GPU with a bit-level implementation of that
// rule for every fp32 input of magnitude below 512 (scaled block values stay
// below 512), both signs.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return (uint32_t)w;
}

// Encode 8 values with a common scale factor into 8 bytes (element 0 lowest).
__device__ __forceinline__ uint2 encode8(const float v[8], float inv) {
  uint2 r;
  r.x = pack4_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  r.y = pack4_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return r;
}

// ------------------------------------------------------- packed MXFP4 weights
//
// A weight matrix W [N rows, K] (E2M1 codes two per byte, low nibble first,
// plus one E8M0 scale per 32 consecutive K) is stored for the GEMM kernels in
// MFMA operand order:
//   codes  [N/64 groups][K/128 steps][4 tiles][64 lanes][16 bytes]
//   scales [N/64 groups][K/128 steps][64 lanes][4 tiles]
// Lane l of tile t in group G and step s holds row  G*64 + pack_row(t, l%16)
// and the 32 elements K in [128 s + 32 (l/16), +32), i.e. exactly the A
// operand of one v_mfma_scale_f32_16x16x128_f8f6f4 with an FP4 A matrix, and
// the scale byte that instruction applies to that lane's K block.  One wave
// step reads 4 KB of codes and 256 B of scales, both contiguous.
//
// pack_row puts the gate/up pair of intermediate column j (rows 2j, 2j+1) and
// the following pairs so that the output lane holding MFMA rows 4q..4q+3 of
// every tile owns the 16 consecutive rows 16q .. 16q+15 of the group.
__device__ __forceinline__ int pack_row(int tile, int m) {
  return 16 * (m >> 2) + 4 * tile + (m & 3);
}

}  // namespace moe
