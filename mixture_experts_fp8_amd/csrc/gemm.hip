// Grouped GEMMs of the A8W4 MoE layer on the gfx950 scaled F8F6F4 MFMA, for
// decode-sized blocks (block_m 16 and 32); larger blocks use gemm_tile.hip.
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
#include "gemm_common.hpp"

namespace moe {

namespace {

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
  if ((int)blockIdx.x >= T) return;
  const int tile = xcd_tile(blockIdx.x, T);
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

  // stage two: the routes' slots and routing weights, fetched before the K
  // loop so the epilogue does not wait for them
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
        const v8i bb = join8(f.b0[c], f.b1[c]);
        acc[0][c] = mfma_fp4_fp8<0>(f.a[0], bb, acc[0][c], f.sa, f.sb[c]);
        acc[1][c] = mfma_fp4_fp8<1>(f.a[1], bb, acc[1][c], f.sa, f.sb[c]);
        acc[2][c] = mfma_fp4_fp8<2>(f.a[2], bb, acc[2][c], f.sa, f.sb[c]);
        acc[3][c] = mfma_fp4_fp8<3>(f.a[3], bb, acc[3][c], f.sa, f.sb[c]);
      }
    }
  };

  // software pipeline: a ring of PD fragments, loads issued PD - 1 steps ahead
  // wave wk of a row group takes steps [wk KS / NWK, (wk + 1) KS / NWK): all
  // KS steps for any KS (a wave may get none when KS < NWK)
  const int s0 = wk * KS / NWK, s1 = (wk + 1) * KS / NWK;
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
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage1_store(part, (int64_t)b * bm + c * 16 + t16, grp, N / 2, g, args.out_q, args.out_s);
      }
    }
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t scr[4][kStage2Scratch];   // one area per wave
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage2_store(part, valid[c] ? slot[c] : -1, wt[c], args, grp, g, scr[wave]);
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

// Blocks of 16 or 32 routes run here; 64 and 128 go to the LDS-tiled kernel.
hipError_t launch_stage1(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16: return launch_gemm<1, 1, MOE_S1_NWK_SMALL, MOE_S1_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 32: return launch_gemm<1, 2, MOE_S1_NWK_SMALL, MOE_S1_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 64:
    case 128: return launch_tile(1, a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

// Stage two splits K over the four waves of a workgroup when K is long (I =
// 2304: 18 steps) and blocks hold at most 16 routes: one wave per row group
// would walk 18 steps of dependent loads, and such a call has too few blocks
// to hide that behind other workgroups (local slice, 1 token: 38 -> 31 us).
// At I = 640 (5 steps), or with blocks of 32, a split measured no gain.
hipError_t launch_stage2(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.bm) {
    case 16:
      return a.K >= 1024 ? launch_gemm<2, 1, 4, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream)
                         : launch_gemm<2, 1, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 32: return launch_gemm<2, 2, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 64:
    case 128: return launch_tile(2, a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
