// Bandwidth-bound kernels of the A8W4 MoE layer: the top-k combine with the
// BF16 output conversion, and the one-time MXFP4 weight packing.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// Top-k combine: out[t, h] = BF16( sum over the token's local slots k, in
// ascending k, of y[t, k, h] ), y holding topk_weight * (w2 h) of each route
// (the routing weight is applied after stage two: aiter PR 5609,
// Configuration) in the route-row format: 16-bit codes plus one exponent
// byte per 32 outputs, decoded exactly to fp32.  One thread per 8
// consecutive outputs; slots whose expert is not local were never written and
// are skipped, so a token with no local route gets zeros.  The fixed
// summation order makes the result bitwise repeatable.  H / 8 is a multiple of
// 64, so the 64 lanes of a wave share one token and its slot mask.
__global__ void __launch_bounds__(256) combine_kernel(const int32_t* __restrict__ ids,
                                                      const int16_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ exps,
                                                      uint16_t* __restrict__ out, int64_t n8,
                                                      int H, int topk, int E, int expert_offset) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int h8 = H / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const int64_t t = __builtin_amdgcn_readfirstlane((int)(i / h8));
    const int h = (int)(i - t * h8) * 8;
    combine8(codes, exps, out, t, h, H, topk, local_slots(ids, t, topk, E, expert_offset));
  }
}

// One thread per (expert, 64-row group, K step, lane): copies the 16-byte K
// block of each of the lane's four tile rows and gathers their four scales.
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ src,
                                                   const uint8_t* __restrict__ src_s,
                                                   uint8_t* __restrict__ dst,
                                                   uint8_t* __restrict__ dst_s, int64_t E,
                                                   int64_t N, int64_t K) {
  const int64_t NG = N / 64, KS = K / 128;
  const int64_t total = E * NG * KS * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int lane = (int)(i & 63);
    int64_t r = i >> 6;
    const int64_t s = r % KS;
    r /= KS;
    const int64_t grp = r % NG;
    const int64_t e = r / NG;
    const int m = lane & 15, g = lane >> 4;
    uint32_t sc = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = grp * 64 + pack_row(t, m);
      const uint8_t* row = src + (e * N + n) * (K / 2);
      const uint4 v = *reinterpret_cast<const uint4*>(row + 64 * s + 16 * g);
      *reinterpret_cast<uint4*>(dst + (((e * NG + grp) * KS + s) * 4 + t) * 1024 + lane * 16) = v;
      sc |= (uint32_t)src_s[(e * N + n) * (K / 32) + 4 * s + g] << (8 * t);
    }
    *reinterpret_cast<uint32_t*>(dst_s + (((e * NG + grp) * KS + s) * 64 + lane) * 4) = sc;
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_combine(int64_t M, int32_t H, int32_t topk, int32_t E, int32_t expert_offset,
                          const int32_t* ids, const int16_t* y_codes, const uint8_t* y_exps,
                          uint16_t* out, hipStream_t stream) {
  const int64_t n8 = M * H / 8;
  if (n8 == 0) return hipSuccess;
  // one thread per 8 outputs, up to 65536 workgroups (the 4096 of the
  // packing kernel left a prefill-shared 16384-token combine 6 % slower:
  // 237 -> 222 us)
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, y_codes, y_exps,
                     out, n8, H, topk, E, expert_offset);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* src, const uint8_t* src_s, uint8_t* dst, uint8_t* dst_s,
                       int64_t E, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t total = E * (N / 64) * (K / 128) * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, src, src_s, dst,
                     dst_s, E, N, K);
  return hipGetLastError();
}

}  // namespace moe
