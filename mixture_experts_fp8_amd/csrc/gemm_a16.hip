// The A16W4 variant of the MoE layer's two grouped GEMMs on gfx950: BF16
// activations times MXFP4 weights (aiter PR 6286, "Retune gfx942 a16w4 DSv4.1
// tiles for Triton 3.8": moe_gemm_a16w4, w1 with apply_swiglu, w2 separate,
// BF16, MXFP4).  Stage one: w13[e] (interleaved gate/up rows) times the routed
// tokens' BF16 rows, SiLU(gate) * up, rounded to a BF16 intermediate.  Stage
// two: w2[e] times that intermediate, scaled by the routing weight, written
// as route rows for the top-k combine shared with the A8W4 layer.
//
// There is no mixed BF16 x FP4 matrix instruction, so each wave converts its
// packed FP4 weight fragment to BF16 with the scaled conversion
// v_cvt_scalef32_pk_bf16_fp4 (two elements per instruction, times the block's
// E8M0 scale: exact for every scale whose products stay normal in BF16) and
// feeds v_mfma_f32_16x16x32_bf16.  Mapping as in gemm.hip ("swap-AB"):
// weights are the A matrix, tokens the B matrix, a wave owns 64 weight rows
// (4 tiles of 16) and the block's bm tokens; a wave step covers 128 K.  This
// file runs blocks of 16 routes (decode sizes); larger blocks run the
// LDS-tiled form of the variant in gemm_tile.hip.
//
// K inside a step: lane l of the packed weights holds the 32 elements
// K [32 (l/16), +32) of its row.  MFMA j (j = 0..3) of the step takes
// elements 8j .. 8j+7 of them, so its lane group q = l/16 covers K
// 32q + 8j + [0, 8); the B operand is loaded with the same assignment (a
// lane reads 64 contiguous bytes of its token row per step), and the sum
// over K is the same dot product in another order.
#include "gemm_common.hpp"

namespace moe {

namespace {

template <int NCG>
struct FragA16 {
  v4i a[4];          // weight codes of the 4 tiles, 32 FP4 each
  uint32_t sa;       // the 4 tiles' E8M0 scale bytes
  v4i b[NCG][4];     // token row K [32 (l/16) + 8j, +8) for j = 0..3, 8 BF16 each
};

// STAGE 1 or 2; NCG column groups of 16 tokens; NWK waves splitting K
// (4 / NWK row groups per workgroup); a ring of PD fragments per wave.
// args.bq: stage 1 the BF16 hidden rows [M, K], stage 2 the BF16
// intermediate [capacity, K] in sorted-row order; args.out_q: stage 1's
// intermediate output.  Weights stream with non-temporal loads.
template <int STAGE, int NCG, int NWK, int PD>
__global__ void __launch_bounds__(256) a16_kernel(GemmArgs args) {
  constexpr int NWR = 4 / NWK;
  const int N = args.N, K = args.K, bm = args.bm, M = args.M;
  const int KS = K / 128;
  const int NG = N / (NWR * 64);
  const int nblk = *args.num_padded / bm;
  const int T = nblk * NG;
  if ((int)blockIdx.x >= T) return;
  const int tile = xcd_tile(blockIdx.x, T);
  const int b = tile / NG, wgg = tile - b * NG;
  const int e = args.block_expert[b];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave / NWK, wk = wave - wr * NWK;
  const int grp = wgg * NWR + wr;
  const int t16 = lane & 15, g = lane >> 4;

  const int32_t* ids = args.sorted_ids + (int64_t)b * bm;
  int rid[NCG];
  bool valid[NCG];
  const uint8_t* brow[NCG];
  int nact = 0;
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    rid[c] = ids[c * 16 + t16];
    valid[c] = rid[c] != M;
    if (__ballot(valid[c]) != 0) nact = c + 1;
    const int64_t row = (STAGE == 1) ? (int64_t)(rid[c] & 0xFFFFFF) : (int64_t)b * bm + c * 16 + t16;
    brow[c] = args.bq + (row * K + 32 * g) * 2;
  }
  int64_t slot[NCG];
  float wt[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    slot[c] = 0;
    wt[c] = 0.f;
    if (STAGE == 2 && valid[c]) {
      slot[c] = route_slot(rid[c], args.topk);
      wt[c] = args.topk_weights[slot[c]];
    }
  }

  const uint8_t* wp = args.w + (int64_t)e * ((int64_t)N * K / 2) + (int64_t)grp * KS * 4096 + lane * 16;
  const uint8_t* wsp = args.ws + (int64_t)e * ((int64_t)N * K / 32) + (int64_t)grp * KS * 256 + lane * 4;

  v4f acc[4][NCG];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < NCG; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

  auto load = [&](FragA16<NCG>& f, int s) {
    const uint8_t* w = wp + (int64_t)s * 4096;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(w + t * 1024));
    f.sa = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsp + (int64_t)s * 256));
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          f.b[c][j] = valid[c] ? *reinterpret_cast<const v4i*>(brow[c] + s * 256 + 16 * j) : v4i{0, 0, 0, 0};
      }
    }
  };
  auto compute = [&](const FragA16<NCG>& f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float sc = e8m0_to_f32((f.sa >> (8 * t)) & 0xFFu);
      const uint32_t wv[4] = {(uint32_t)f.a[t].x, (uint32_t)f.a[t].y, (uint32_t)f.a[t].z, (uint32_t)f.a[t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 a = fp4x8_to_bf16(wv[j], sc);
#pragma unroll
        for (int c = 0; c < NCG; ++c)
          if (c < nact)
            acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, f.b[c][j]),
                                                                acc[t][c], 0, 0, 0);
      }
    }
  };

  const int s0 = wk * KS / NWK, s1 = (wk + 1) * KS / NWK;
  FragA16<NCG> f[PD];
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
    // partial sums of waves wk = 1 .. NWK-1 added to wave 0's in that order
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
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        a16_stage1_store(part, (int64_t)b * bm + c * 16 + t16, grp, N / 2, g,
                         reinterpret_cast<uint16_t*>(args.out_q));
      }
    }
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t scr[4][kStage2Scratch];
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage2_store(part, valid[c] ? slot[c] : -1, wt[c], args, grp, g, scr[wave]);
      }
    }
  }
}

template <int STAGE, int NCG, int NWK>
hipError_t launch_a16_t(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  constexpr int NWR = 4 / NWK;
  const int64_t grid = max_blocks * (a.N / (NWR * 64));
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((a16_kernel<STAGE, NCG, NWK, 2>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Blocks of 16 run here: stage one splits K (H) over the four waves, as the
// A8W4 decode kernel does, stage two keeps one wave per row group (K = I, a
// few steps).  Blocks of 32, 64 and 128 run the LDS-tiled kernel
// (gemm_tile.hip): 384 experts top-6, 1536 tokens in blocks of 32 647 us here
// against 541 us there, 4096 tokens in blocks of 64 1346 against 838.
hipError_t launch_a16_stage1(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16: return launch_a16_t<1, 1, 4>(a, max_blocks, stream);
    case 32:
    case 64:
    case 128: return launch_a16_tile(1, a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_a16_stage2(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16: return launch_a16_t<2, 1, 1>(a, max_blocks, stream);
    case 32:
    case 64:
    case 128: return launch_a16_tile(2, a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
