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
// exponent field of their largest magnitude (as fp32), at least 14.  Output
// v (the routing weight times the fp32 accumulator, an exact product) is
// stored as the 16-bit integer RNE(v * 2^(140 - S)), which lies in [-2^14, 2^14],
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

// The code of x * m (|x m| <= 2^14) in the low 16 bits of the result: one
// fused multiply-add onto 1.5 * 2^23 rounds the exact product to the nearest
// integer, ties to even (the sum's unit in the last place is 1), and leaves
// it as a two's-complement offset in the low mantissa bits.
__device__ __forceinline__ uint32_t route_code_bits(float x, float m) {
  return __float_as_uint(__builtin_fmaf(x, m, 12582912.0f));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> BF16 bits, nearest with ties to even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ----------------------------------------------- hand-over between workgroups
//
// Data one workgroup hands to another inside a launch (the fused decode
// launch) goes through loads and stores that are coherent across the XCDs at
// device scope with no cache maintenance: agent-scope relaxed atomics, which
// gfx950 issues with the sc1 cache policy (written through to, and read back
// from, the level all XCDs share).  Cache-wide release/acquire fences (L2
// write-back and invalidate) cost far more when hundreds of workgroups use
// them.  COH = false gives ordinary accesses.
template <bool COH>
__device__ __forceinline__ void st64(void* p, uint64_t v) {
  if constexpr (COH) __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<uint64_t*>(p) = v;
}
template <bool COH>
__device__ __forceinline__ void st16(void* p, uint16_t v) {
  if constexpr (COH) __hip_atomic_store(static_cast<uint16_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<uint16_t*>(p) = v;
}
template <bool COH>
__device__ __forceinline__ void st8(void* p, uint8_t v) {
  if constexpr (COH) __hip_atomic_store(static_cast<uint8_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<uint8_t*>(p) = v;
}
template <bool COH>
__device__ __forceinline__ void st128(void* p, v4i v) {
  if constexpr (COH) {
    st64<true>(p, (uint64_t)(uint32_t)v.x | ((uint64_t)(uint32_t)v.y << 32));
    st64<true>(static_cast<uint8_t*>(p) + 8, (uint64_t)(uint32_t)v.z | ((uint64_t)(uint32_t)v.w << 32));
  } else {
    *static_cast<v4i*>(p) = v;
  }
}
// The aligned 4 bytes holding byte p, with byte p at bit 8 (p & 3).  (A
// coherent single-byte load would be zero-extended by an instruction right
// behind it, which waits for every load in flight; the caller extracts the
// byte where it is used instead.)
template <bool COH>
__device__ __forceinline__ uint32_t ld_word_of(const uint8_t* p) {
  uint32_t* q = reinterpret_cast<uint32_t*>((uintptr_t)p & ~(uintptr_t)3);
  if constexpr (COH) return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *q;
}
__device__ __forceinline__ uint32_t byte_of(uint32_t word, const uint8_t* p) {
  return (word >> (8 * ((uintptr_t)p & 3))) & 0xFFu;
}
// 16 bytes; NT: non-temporal when not coherent
template <bool COH, bool NT = false>
__device__ __forceinline__ v4i ld128(const void* p) {
  if constexpr (COH) {
    uint64_t* q = static_cast<uint64_t*>(const_cast<void*>(p));
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v4i{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
  } else if constexpr (NT) {
    return __builtin_nontemporal_load(static_cast<const v4i*>(p));
  } else {
    return *static_cast<const v4i*>(p);
  }
}

// Waits until every memory operation this wave has issued is complete (its
// stores performed where ld/st with COH read them), before anything after it
// is issued; the signal fences keep the compiler from moving memory accesses
// across the wait.
__device__ __forceinline__ void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Mask of a token's local slots: bit k set when topk_ids[t, k] names one of
// the E experts held here (global ids expert_offset .. expert_offset + E - 1).
__device__ __forceinline__ unsigned local_slots(const int32_t* ids, int64_t t, int topk, int E,
                                                int expert_offset) {
  unsigned mask = 0;
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k)
    if (k < topk && (unsigned)(ids[t * topk + k] - expert_offset) < (unsigned)E) mask |= 1u << k;
  return mask;
}

// Top-k combine of 8 consecutive outputs h .. h+7 of token t: BF16 (nearest
// even) of the float32 sum, in ascending k over the slots in mask, of the
// decoded route rows.  Each code decodes exactly (a 15-bit integer times a
// power of two), so the sum does not depend on instruction selection; all of
// the token's loads are issued before the first add.
// COH: the route rows come from other workgroups of the same launch.
template <bool COH = false>
__device__ __forceinline__ void combine8(const int16_t* __restrict__ codes,
                                         const uint8_t* __restrict__ exps, uint16_t* __restrict__ out,
                                         int64_t t, int h, int H, int topk, unsigned mask) {
  v4i c[kMaxTopk];
  uint32_t sw[kMaxTopk];
  const uint8_t* ex = exps + t * topk * (H / 32) + h / 32;
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    if (mask & (1u << k)) {
      c[k] = ld128<COH, true>(codes + (t * topk + k) * H + h);
      sw[k] = ld_word_of<COH>(ex + k * (H / 32));
    }
  }
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    if (mask & (1u << k)) {
      const float m = route_decode_mul((int)byte_of(sw[k], ex + k * (H / 32)));
      const int w[4] = {c[k].x, c[k].y, c[k].z, c[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // code * 2^(S - 140) is exact, so the product rounds nothing
        a[2 * j] += (float)(int16_t)(w[j] & 0xFFFF) * m;
        a[2 * j + 1] += (float)(w[j] >> 16) * m;
      }
    }
  }
  uint4 r;
  r.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
  r.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
  r.z = f32_to_bf16(a[4]) | (f32_to_bf16(a[5]) << 16);
  r.w = f32_to_bf16(a[6]) | (f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(out + t * H + h) = r;
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
