// The matrix instructions the grouped GEMMs are built from, one instruction
// per 16 x 16 output tile, exported so that tests can measure them against
// exact arithmetic: the scaled FP4 x FP8 MFMA of the A8W4 layer (operand
// layout, scale-byte selection, the error of its internal accumulation,
// which sets the local error budget of the requantised intermediate) and the
// BF16 MFMA of the A16W4 variant; and the weight-streaming probe behind the
// packed weight layout.
#include "gemm_common.hpp"

namespace moe {

namespace {

// One wave per tile i:
//   A  [16 rows][64 bytes]  E2M1 codes, K = 128, element 2c in the low nibble
//   as [16 rows][4]         E8M0 scale of each row's K blocks of 32
//   B  [16 cols][128 bytes] E4M3 codes
//   bs [16 cols][4]         E8M0 scale of each column's K blocks of 32
//   D  [16 rows][16 cols]   float32, from a zero accumulator
// The scale bytes reach the instruction as byte SEL of their 32-bit operand
// (the other bytes hold 0xFF, an invalid scale); the B scale is byte 0 of its
// operand, the others 0xFF likewise.  So the byte selection is checked too.
template <int SEL>
__global__ void __launch_bounds__(64) mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ as,
                                                        const uint8_t* __restrict__ b,
                                                        const uint8_t* __restrict__ bs,
                                                        float* __restrict__ d) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
  const uint8_t* ai = a + i * 16 * 64;
  const uint8_t* bi = b + i * 16 * 128;
  // A lane (m, g): row m, K [32 g, +32) = 16 bytes at 16 g
  const v4i av = *reinterpret_cast<const v4i*>(ai + m * 64 + 16 * g);
  // B lane (n, g): column n, K [16 g, +16) and [64 + 16 g, +16)
  const v4i b0 = *reinterpret_cast<const v4i*>(bi + m * 128 + 16 * g);
  const v4i b1 = *reinterpret_cast<const v4i*>(bi + m * 128 + 64 + 16 * g);
  // scale of lane group g: K block g of row / column m
  const uint32_t sa = (0xFFFFFFFFu & ~(0xFFu << (8 * SEL))) | ((uint32_t)as[i * 64 + m * 4 + g] << (8 * SEL));
  const uint32_t sb = 0xFFFFFF00u | (uint32_t)bs[i * 64 + m * 4 + g];
  const v4f acc = mfma_fp4_fp8<SEL>(av, join8(b0, b1), v4f{0.f, 0.f, 0.f, 0.f}, sa, sb);
  // D lane (n, g): column n, rows 4 g .. 4 g + 3
#pragma unroll
  for (int r = 0; r < 4; ++r) d[i * 256 + (4 * g + r) * 16 + m] = acc[r];
}

// The BF16 instruction of the A16W4 variant (v_mfma_f32_16x16x32_bf16), one
// wave per tile i: A [16 rows][32] and B [16 cols][32] BF16, D [16][16]
// float32 from a zero accumulator.  A lane (m, g) holds row m, K [8 g, +8);
// B lane (n, g) column n, K [8 g, +8); D lane (n, g) column n, rows 4 g .. +3.
__global__ void __launch_bounds__(64) mfma_bf16_probe_kernel(const uint16_t* __restrict__ a,
                                                             const uint16_t* __restrict__ b,
                                                             float* __restrict__ d) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
  const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4i*>(a + i * 512 + m * 32 + 8 * g));
  const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4i*>(b + i * 512 + m * 32 + 8 * g));
  const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) d[i * 256 + (4 * g + r) * 16 + m] = acc[r];
}

// Weight streaming in the decode stage-one kernel's shape (one workgroup per
// 64-row group, 4 waves splitting K, non-temporal 16-byte loads, every lane
// loading exactly the A operand of one MFMA tile per K step), from the
// packed layout of moe_a8w4_pack_weights (1 KB contiguous per instruction)
// or from the raw row-major MXFP4 layout [rows, K/2] (each instruction 16
// rows x 64 B).  Lane (m, q) of tile t at step s holds row
// 64 G + pack_row(t, m), K [128 s + 32 q, +32), and the tile's E8M0 scale
// as byte t of one word, in both kernels; each lane folds what it loads into
// one word, and a wave writes that word of lane 0 ... 63 summed: for raw
// weights and their packed form the two kernels write the same words.
template <bool PACKED>
__global__ void __launch_bounds__(256) stream_probe_kernel(const uint8_t* __restrict__ w,
                                                           const uint8_t* __restrict__ ws, int K,
                                                           uint32_t* __restrict__ out) {
  const int64_t G = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int KS = K / 128;
  const int s0 = wave * KS / 4, s1 = (wave + 1) * KS / 4;
  uint32_t acc = 0;
  for (int s = s0; s < s1; ++s) {
    v4i a[4];
    uint32_t sc = 0;
    if constexpr (PACKED) {
      const uint8_t* base = w + (G * KS + s) * 4096 + lane * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + t * 1024));
      sc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ws + ((G * KS + s) * 64 + lane) * 4));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t row = G * 64 + pack_row(t, m);
        a[t] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(w + row * (K / 2) + 64 * s + 16 * q));
        sc |= (uint32_t)ws[row * (K / 32) + 4 * s + q] << (8 * t);
      }
    }
    acc += (uint32_t)(a[0].x ^ a[1].y ^ a[2].z ^ a[3].w) + sc;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) out[G * 4 + wave] = acc;
}

}  // namespace

hipError_t launch_stream_probe(int layout, int64_t groups, int K, const uint8_t* w, const uint8_t* ws,
                               uint32_t* out, hipStream_t stream) {
  if (groups <= 0) return hipSuccess;
  if (layout == 0)
    hipLaunchKernelGGL(stream_probe_kernel<true>, dim3((unsigned)groups), dim3(256), 0, stream, w, ws, K, out);
  else
    hipLaunchKernelGGL(stream_probe_kernel<false>, dim3((unsigned)groups), dim3(256), 0, stream, w, ws, K, out);
  return hipGetLastError();
}

hipError_t launch_mfma_bf16_probe(int64_t n, const uint16_t* a, const uint16_t* b, float* d,
                                  hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_bf16_probe_kernel, dim3((unsigned)n), dim3(64), 0, stream, a, b, d);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int64_t n, int sel, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, float* d, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)n), blk(64);
  switch (sel) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, blk, 0, stream, a, as, b, bs, d); break;
    case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, blk, 0, stream, a, as, b, bs, d); break;
    case 2: hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, blk, 0, stream, a, as, b, bs, d); break;
    default: hipLaunchKernelGGL(mfma_probe_kernel<3>, grid, blk, 0, stream, a, as, b, bs, d); break;
  }
  return hipGetLastError();
}

}  // namespace moe
