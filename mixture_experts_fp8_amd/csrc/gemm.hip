// Grouped GEMMs of the A8W4 MoE layer on the gfx950 scaled F8F6F4 MFMA.
//
// Stage one: for each block of sorted routes of expert e, gate/up rows of
// w13[e] (MXFP4, interleaved: row 2j gate j, row 2j+1 up j) times the routed
// tokens' FP8 activations, SiLU(gate) * up, and per-1x32 FP8 requantisation of
// the intermediate, with no routing weight.  Stage two: w2[e] times that
// intermediate, scaled by the routing weight, written per route (token, slot)
// for the top-k combine.  (aiter PR 5609, "Add DeepSeek V4.1 Flash TP4 gfx950 MoE
// tuning", Configuration: BF16 output, FP8 activations, MXFP4 weights,
// per-1x32 scaling, interleaved gate/up, SiLU, no stage-one routing-weight
// multiplication; aiter PR 5904, "Fused-MoE kernel, expert-parallel
// benchmark": sorting, both stages and the intermediate quantization form one
// call.)
//
// Mapping ("swap-AB"): the weight rows are the MFMA's A matrix (16 rows x 128 K
// of FP4 per instruction, read straight from the packed weight layout, 4 KB
// contiguous per wave step) and the routed tokens are its B matrix (16 columns
// x 128 K of FP8).  A wave owns 64 weight rows (4 tiles) and all bm tokens of
// a block (bm/16 column groups); column groups past the block's last routed
// token are skipped, so decode-sized blocks cost one MFMA column group while
// the weights stream once.  A workgroup is 4 waves: either 4 row groups over
// the whole K, or (small token counts) one row group with K split 4 ways and
// the partial sums added through LDS in a fixed order.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 with A = FP4, B = FP8
// (measured on gfx950): A lane l holds row l%16, K [32(l/16), +32) in 16 bytes
// (low nibble first); B lane l holds column l%16, K [16(l/16), +16) in bytes
// 0..15 and K [64 + 16(l/16), +16) in bytes 16..31; the scale operand of lane
// l applies to K block l/16 of its row/column; the result lane l holds column
// l%16, rows 4(l/16) .. 4(l/16)+3.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_fp8(const v4i& a, const v8i& b, const v4f& c, uint32_t sa,
                                            uint32_t sb) {
  const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  // format codes: A = 4 (FP4 E2M1), B = 0 (FP8 E4M3); OPSEL picks the scale byte of this tile
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, OPSEL, (int)sa, 0, (int)sb);
}

// Weight loads: non-temporal (streamed past the caches) when an expert's
// weights are read once per call, cached when several blocks reuse them.
template <bool NT, typename T>
__device__ __forceinline__ T load_w(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

template <int NCG>
struct Frag {
  v4i a[4];        // weight codes, one 16-byte K block per tile
  uint32_t sa;     // the four tiles' scale bytes
  v4i b0[NCG];     // token codes K [16g, +16)
  v4i b1[NCG];     // token codes K [64 + 16g, +16)
  uint32_t sb[NCG];
};

// STAGE 1 or 2; NCG column groups of 16 tokens (block_m = 16 NCG); NWK waves
// splitting K inside a workgroup (4 / NWK row groups per workgroup); PD steps
// of loads in flight per wave (PD - 1 steps prefetched ahead of the MFMAs);
// NT streams the weights with non-temporal loads.
template <int STAGE, int NCG, int NWK, int PD, bool NT>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs args) {
  constexpr int NWR = 4 / NWK;
  const int N = args.N, K = args.K, bm = args.bm, M = args.M;
  const int KS = K / 128;
  const int NG = N / (NWR * 64);
  const int nblk = *args.num_padded / bm;
  const int T = nblk * NG;
  const int wg = blockIdx.x;
  if (wg >= T) return;
  // XCD-aware order: workgroup 8j + x runs on XCD x; XCD x takes a contiguous
  // run of (block, row group) tiles so that the blocks of one expert share L2.
  const int x = wg & 7, j = wg >> 3;
  const int q8 = T >> 3, rem = T & 7;
  const int tile = x * q8 + (x < rem ? x : rem) + j;
  const int b = tile / NG, wgg = tile - b * NG;
  const int e = args.block_expert[b];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave / NWK, wk = wave - wr * NWK;
  const int grp = wgg * NWR + wr;
  const int t16 = lane & 15, g = lane >> 4;

  // rows of this block seen by this lane (column t16 of each column group)
  const int32_t* ids = args.sorted_ids + (int64_t)b * bm;
  int rid[NCG];
  bool valid[NCG];
  const uint8_t* brow[NCG];
  const uint8_t* bsrow[NCG];
  int nact = 0;
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    rid[c] = ids[c * 16 + t16];
    valid[c] = rid[c] != M;
    if (__ballot(valid[c]) != 0) nact = c + 1;
    const int64_t row = (STAGE == 1) ? (int64_t)(rid[c] & 0xFFFFFF) : (int64_t)b * bm + c * 16 + t16;
    brow[c] = args.bq + row * K + 16 * g;
    bsrow[c] = args.bs + row * (K / 32) + g;
  }

  const uint8_t* wp = args.w + (int64_t)e * ((int64_t)N * K / 2) + (int64_t)grp * KS * 4096 + lane * 16;
  const uint8_t* wsp = args.ws + (int64_t)e * ((int64_t)N * K / 32) + (int64_t)grp * KS * 256 + lane * 4;

  v4f acc[4][NCG];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < NCG; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

  auto load = [&](Frag<NCG>& f, int s) {
    const uint8_t* w = wp + (int64_t)s * 4096;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = load_w<NT, v4i>(w + t * 1024);
    f.sa = load_w<NT, uint32_t>(wsp + (int64_t)s * 256);
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        if (valid[c]) {
          f.b0[c] = *reinterpret_cast<const v4i*>(brow[c] + s * 128);
          f.b1[c] = *reinterpret_cast<const v4i*>(brow[c] + s * 128 + 64);
          f.sb[c] = bsrow[c][4 * s];
        } else {
          f.b0[c] = v4i{0, 0, 0, 0};
          f.b1[c] = v4i{0, 0, 0, 0};
          f.sb[c] = 127u;
        }
      }
    }
  };
  auto compute = [&](const Frag<NCG>& f) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v8i bb = {f.b0[c].x, f.b0[c].y, f.b0[c].z, f.b0[c].w,
                        f.b1[c].x, f.b1[c].y, f.b1[c].z, f.b1[c].w};
        acc[0][c] = mfma_fp4_fp8<0>(f.a[0], bb, acc[0][c], f.sa, f.sb[c]);
        acc[1][c] = mfma_fp4_fp8<1>(f.a[1], bb, acc[1][c], f.sa, f.sb[c]);
        acc[2][c] = mfma_fp4_fp8<2>(f.a[2], bb, acc[2][c], f.sa, f.sb[c]);
        acc[3][c] = mfma_fp4_fp8<3>(f.a[3], bb, acc[3][c], f.sa, f.sb[c]);
      }
    }
  };

  // software pipeline: a ring of PD fragments, loads issued PD - 1 steps ahead
  const int s0 = wk * (KS / NWK), s1 = s0 + KS / NWK;
  Frag<NCG> f[PD];
#pragma unroll
  for (int u = 0; u < PD - 1; ++u)
    if (s0 + u < s1) load(f[u], s0 + u);
  for (int s = s0; s < s1; s += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (s + u >= s1) break;
      if (s + u + PD - 1 < s1) load(f[(u + PD - 1) % PD], s + u + PD - 1);
      compute(f[u]);
    }
  }

  if constexpr (NWK > 1) {
    // partial sums of waves wk = 1 .. NWK-1 are added to wave 0's in that order
    __shared__ float red[(NWK - 1) * NWR][4][NCG][4][64];
    if (wk > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < NCG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(wk - 1) * NWR + wr][t][c][r][lane] = acc[t][c][r];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int p = 0; p < NWK - 1; ++p)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < NCG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][c][r] += red[p * NWR + wr][t][c][r][lane];
  }

  if constexpr (STAGE == 1) {
    // lane (t16, g) holds rows 16g + 4t + r of the group: gate/up of the eight
    // intermediate columns 32*grp + 8g + (2t + r/2); the group's 32 columns are
    // one quantisation block, spread over the four lanes with equal t16.
    const int I = N / 2;
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        float h[8];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float gate = acc[t][c][2 * q], up = acc[t][c][2 * q + 1];
            h[2 * t + q] = gate / (1.0f + __expf(-gate)) * up;
          }
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(h[q]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int E = block_exponent(amax);
        const uint2 codes = encode8(h, exp2_neg(E));
        const int64_t p = (int64_t)b * bm + c * 16 + t16;
        *reinterpret_cast<uint2*>(args.out_q + p * I + grp * 32 + 8 * g) = codes;
        if (g == 0) args.out_s[p * (I / 32) + grp] = (uint8_t)(E + 127);
      }
    }
  } else {
    // lane (t16, g) holds output columns 64*grp + 16g + 4t + r of its route:
    // 16 consecutive floats, so the four lanes of a route write 256 B in a row
    const int H = N;
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact && valid[c]) {
        const int tok = rid[c] & 0xFFFFFF, k = rid[c] >> kSentinelShift;
        const int64_t slot = (int64_t)tok * args.topk + k;
        const float wt = args.topk_weights[slot];
        float4* dst = reinterpret_cast<float4*>(args.y_routes + slot * H + grp * 64 + 16 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          dst[t] = make_float4(wt * acc[t][c][0], wt * acc[t][c][1], wt * acc[t][c][2], wt * acc[t][c][3]);
      }
    }
  }
}

template <int STAGE, int NCG, int NWK, int PD, bool NT>
hipError_t launch_gemm(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  constexpr int NWR = 4 / NWK;
  const int64_t NG = a.N / (NWR * 64);
  const int64_t grid = max_blocks * NG;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<STAGE, NCG, NWK, PD, NT>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

#ifndef MOE_S1_PD
#define MOE_S1_PD 2
#endif
#ifndef MOE_S2_PD
#define MOE_S2_PD 2
#endif
#ifndef MOE_S1_NWK_SMALL
#define MOE_S1_NWK_SMALL 4
#endif
#ifndef MOE_NT_SMALL
#define MOE_NT_SMALL true
#endif

}  // namespace

hipError_t launch_stage1(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16: return launch_gemm<1, 1, MOE_S1_NWK_SMALL, MOE_S1_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 32: return launch_gemm<1, 2, MOE_S1_NWK_SMALL, MOE_S1_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 64: return launch_gemm<1, 4, 1, 2, false>(a, max_blocks, stream);
    case 128: return launch_gemm<1, 8, 1, 2, false>(a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stage2(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16: return launch_gemm<2, 1, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 32: return launch_gemm<2, 2, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 64: return launch_gemm<2, 4, 1, 2, false>(a, max_blocks, stream);
    case 128: return launch_gemm<2, 8, 1, 2, false>(a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
