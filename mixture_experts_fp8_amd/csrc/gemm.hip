// Grouped GEMMs of the A8W4 MoE layer on the gfx950 scaled F8F6F4 MFMA, for
// decode-sized blocks (block_m 16 and 32); larger blocks use gemm_tile.hip.
//
// Stage one: for each block of sorted routes of expert e, gate/up rows of
// w13[e] (MXFP4, interleaved: row 2j gate j, row 2j+1 up j) times the routed
// tokens' FP8 activations, SiLU(gate) * up, and per-1x32 FP8 requantisation of
// the intermediate, with no routing weight.  Stage two: w2[e] times that
// intermediate, scaled by the routing weight, written per route (token, slot)
// for the top-k combine.  (The layer's definition: aiter PR 5609, "Add
// DeepSeek V4.1 Flash TP4 gfx950 MoE tuning", Configuration; the span of one
// call: aiter PR 5904, "Fused-MoE kernel, expert-parallel benchmark".)
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
  uint32_t sb[NCG];  // token scale byte (fused stage two: the aligned word holding it)
};

// Bytes of LDS one tile needs: the split-K partial sums, then (stage two)
// one stage2_store scratch area per wave, then (fused stage two) the list of
// tokens whose combine falls to this workgroup.
template <int STAGE, int NCG, int NWK>
constexpr int tile_smem_bytes() {
  return (NWK - 1) * (4 / NWK) * 4 * NCG * 4 * 64 * 4 + (STAGE == 2 ? 4 * kStage2Scratch + 2 * 32 * 4 : 0);
}

// Longest wait of a fused stage-two tile for its block's stage one, in polls
// (each a device-scope load plus s_sleep 8, 512 clocks): about half a second.
// Only reached if the workgroups it waits for never run; the tile then
// records it in the status word and goes on, so the launch always ends.
constexpr int kSpinLimit = 1 << 19;

// One tile: stage STAGE for (sorted block, row group of the weights) number
// wg of T = blocks * NG, mapped XCD-aware.  NCG column groups of 16 tokens
// (block_m = 16 NCG); NWK waves splitting K inside the workgroup (4 / NWK
// row groups per workgroup); PD steps of loads in flight per wave (PD - 1
// steps prefetched ahead of the MFMAs); NT streams the weights with
// non-temporal loads.  FUSED: part of the fused decode launch -- a stage-one
// tile counts itself done for its block, a stage-two tile first waits for its
// block's stage one (its first weight steps already loading) and afterwards
// runs the top-k combine of each token whose last route it completed.
template <int STAGE, int NCG, int NWK, int PD, bool NT, bool FUSED>
__device__ __forceinline__ void run_tile(const GemmArgs& args, const FusedArgs& fa, int wg,
                                         uint8_t* smem) {
  constexpr int NWR = 4 / NWK;
  const int N = args.N, K = args.K, bm = args.bm, M = args.M;
  const int KS = K / 128;
  const int NG = N / (NWR * 64);
  const int nblk = *args.num_padded / bm;
  const int T = nblk * NG;
  if (wg >= T) return;
  const int tile = xcd_tile(wg, T);
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
  int sbsh[NCG];   // bit position of the token scale byte in its aligned word
  int nact = 0;
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    rid[c] = ids[c * 16 + t16];
    valid[c] = rid[c] != M;
    if (__ballot(valid[c]) != 0) nact = c + 1;
    const int64_t row = (STAGE == 1) ? (int64_t)(rid[c] & 0xFFFFFF) : (int64_t)b * bm + c * 16 + t16;
    brow[c] = args.bq + row * K + 16 * g;
    bsrow[c] = args.bs + row * (K / 32) + g;
    sbsh[c] = 8 * (int)((uintptr_t)bsrow[c] & 3);
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
  // fused stage two: thread i < bm follows route i of the block through the
  // combine: its token, and that token's local slots
  int my_tok = -1;
  unsigned my_mask = 0;
  if constexpr (FUSED && STAGE == 2) {
    if ((int)threadIdx.x < bm) {
      const int r = ids[threadIdx.x];
      if (r != M) {
        my_tok = r & 0xFFFFFF;
        my_mask = local_slots(fa.topk_ids, my_tok, args.topk, fa.num_experts, fa.expert_offset);
      }
    }
  }

  const uint8_t* wp = args.w + (int64_t)e * ((int64_t)N * K / 2) + (int64_t)grp * KS * 4096 + lane * 16;
  const uint8_t* wsp = args.ws + (int64_t)e * ((int64_t)N * K / 32) + (int64_t)grp * KS * 256 + lane * 4;

  v4f acc[4][NCG];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < NCG; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](Frag<NCG>& f, int s) {
    const uint8_t* w = wp + (int64_t)s * 4096;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = load_w<NT, v4i>(w + t * 1024);
    f.sa = load_w<NT, uint32_t>(wsp + (int64_t)s * 256);
  };
  // fused stage two reads the intermediate other workgroups of the launch wrote
  constexpr bool COH = FUSED && STAGE == 2;
  auto load_b = [&](Frag<NCG>& f, int s) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        if (valid[c]) {
          f.b0[c] = ld128<COH>(brow[c] + s * 128);
          f.b1[c] = ld128<COH>(brow[c] + s * 128 + 64);
          // fused: the word holding the scale byte, extracted in compute()
          // (steps move by 4 bytes, so its position stays sbsh[c])
          if constexpr (COH) f.sb[c] = ld_word_of<true>(bsrow[c] + 4 * s);
          else f.sb[c] = bsrow[c][4 * s];
        } else {
          f.b0[c] = v4i{0, 0, 0, 0};
          f.b1[c] = v4i{0, 0, 0, 0};
          f.sb[c] = 0x7F7F7F7Fu;
        }
      }
    }
  };
  auto compute = [&](const Frag<NCG>& f) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v8i bb = join8(f.b0[c], f.b1[c]);
        const uint32_t sb = COH ? (f.sb[c] >> sbsh[c]) & 0xFFu : f.sb[c];
        acc[0][c] = mfma_fp4_fp8<0>(f.a[0], bb, acc[0][c], f.sa, sb);
        acc[1][c] = mfma_fp4_fp8<1>(f.a[1], bb, acc[1][c], f.sa, sb);
        acc[2][c] = mfma_fp4_fp8<2>(f.a[2], bb, acc[2][c], f.sa, sb);
        acc[3][c] = mfma_fp4_fp8<3>(f.a[3], bb, acc[3][c], f.sa, sb);
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
    if (s0 + u < s1) load_a(f[u], s0 + u);
  if constexpr (FUSED && STAGE == 2) {
    // the block's intermediate is complete once all of its stage-one tiles
    // have counted themselves, each after its stores were performed; it is
    // then read with device-scope loads (load_b), so no cache maintenance
    // is needed.  Each block's counter has a 256-byte run of its own, and
    // the polls back off, so waiting tiles do not crowd one memory channel.
    if (threadIdx.x == 0) {
      int* done = fa.block_done + (int64_t)b * kCounterStride;
      int it = 0;
      while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < fa.ng1) {
        if (++it == kSpinLimit) {
          __hip_atomic_store(fa.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < PD - 1; ++u)
    if (s0 + u < s1) load_b(f[u], s0 + u);
  for (int s = s0; s < s1; s += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (s + u >= s1) break;
      if (s + u + PD - 1 < s1) {
        load_a(f[(u + PD - 1) % PD], s + u + PD - 1);
        load_b(f[(u + PD - 1) % PD], s + u + PD - 1);
      }
      compute(f[u]);
    }
  }

  // waves wk > 0 hand their partial sums to wave wk = 0 of their row group,
  // which alone runs the epilogue
  constexpr bool keep_all = FUSED && STAGE == 2;   // the combine below needs every wave
  if constexpr (NWK > 1) {
    // partial sums of waves wk = 1 .. NWK-1 are added to wave 0's in that order
    float(*red)[4][NCG][4][64] = reinterpret_cast<float(*)[4][NCG][4][64]>(smem);
    if (wk > 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < NCG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(wk - 1) * NWR + wr][t][c][r][lane] = acc[t][c][r];
    }
    __syncthreads();
    if (wk > 0 && !keep_all) return;
    if (wk == 0) {
#pragma unroll
      for (int p = 0; p < NWK - 1; ++p)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c = 0; c < NCG; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][c][r] += red[p * NWR + wr][t][c][r][lane];
    }
  }

  if constexpr (STAGE == 1) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage1_store<FUSED>(part, (int64_t)b * bm + c * 16 + t16, grp, N / 2, g, args.out_q, args.out_s);
      }
    }
    if constexpr (FUSED) {
      // NWK = 4: wave 0 alone wrote this tile's rows (device-scope stores);
      // once they are performed, count the tile done
      static_assert(NWK == 4, "fused stage one expects one row group per workgroup");
      wait_memory();
      if (lane == 0)
        __hip_atomic_fetch_add(fa.block_done + (int64_t)b * kCounterStride, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    uint8_t* scr = smem + (NWK - 1) * NWR * 4 * NCG * 4 * 64 * 4 + wave * kStage2Scratch;
    if (wk == 0) {
#pragma unroll
      for (int c = 0; c < NCG; ++c) {
        if (c < nact) {
          const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
          stage2_store<FUSED>(part, valid[c] ? slot[c] : -1, wt[c], args, grp, g, scr);
        }
      }
    }
    if constexpr (FUSED) {
      // route rows of this tile (output columns [W wgg, W (wgg + 1)), W = 64
      // NWR), written with device-scope stores, are performed; each route
      // counts itself for its token, and the route that completes a token's
      // count (one per local slot) makes this workgroup run that token's
      // combine over these columns.  Thread 64 counts the tile for its
      // block; the block's last stage-two tile clears the block's counters
      // (every tile of the block is past its wait by then).
      constexpr int W = NWR * 64;
      int* list_tok = reinterpret_cast<int*>(smem + (NWK - 1) * NWR * 4 * NCG * 4 * 64 * 4 + 4 * kStage2Scratch);
      unsigned* list_mask = reinterpret_cast<unsigned*>(list_tok + 32);
      wait_memory();
      __syncthreads();
      if ((int)threadIdx.x < bm) {
        int t = -1;
        if (my_tok >= 0) {
          int* cnt = fa.token_done + (int64_t)my_tok * NG + wgg;
          const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (old == __builtin_popcount(my_mask) - 1) {
            t = my_tok;
            __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        list_tok[threadIdx.x] = t;
        list_mask[threadIdx.x] = my_mask;
      } else if (threadIdx.x == 64) {
        const int seen = __hip_atomic_fetch_add(fa.block_seen + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen == NG - 1) {
          __hip_atomic_store(fa.block_done + (int64_t)b * kCounterStride, 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(fa.block_seen + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
      for (int i = wave; i < bm; i += 4) {
        const int t = list_tok[i];
        if (t < 0) continue;
        if (lane < W / 8)
          combine8<true>(args.y_codes, args.y_exps, fa.out, t, wgg * W + 8 * lane, N, args.topk, list_mask[i]);
      }
    }
  }
}

template <int STAGE, int NCG, int NWK, int PD, bool NT>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[tile_smem_bytes<STAGE, NCG, NWK>()];
  run_tile<STAGE, NCG, NWK, PD, NT, false>(args, FusedArgs{}, blockIdx.x, smem);
}

// The fused decode launch: stage one, stage two and the top-k combine of one
// call.  Workgroups [0, g1) run stage-one tiles, [g1, g1 + g2) stage-two
// tiles, the rest write the zero rows of tokens without a local route.
// Deadlock freedom: a stage-two tile waits only for stage-one tiles, which
// never wait, and every stage-one workgroup precedes every stage-two one in
// workgroup order; workgroups are dispatched in order, so whenever a
// stage-two tile waits, the tiles it waits for are running or done.  (The
// wait is bounded besides, see kSpinLimit.)
template <int NCG, int NWK2, int PD1, int PD2>
__global__ void __launch_bounds__(256) fused_kernel(GemmArgs a1, GemmArgs a2, FusedArgs fa) {
  constexpr int S1 = tile_smem_bytes<1, NCG, 4>(), S2 = tile_smem_bytes<2, NCG, NWK2>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[S1 > S2 ? S1 : S2];
  const int wg = blockIdx.x;
  if (wg < fa.g1) {
    run_tile<1, NCG, 4, PD1, true, true>(a1, fa, wg, smem);
  } else if (wg < fa.g1 + fa.g2) {
    run_tile<2, NCG, NWK2, PD2, true, true>(a2, fa, wg - fa.g1, smem);
  } else {
    // one wave per token: zeros for a token none of whose slots is local
    const int64_t t = (int64_t)(wg - fa.g1 - fa.g2) * 4 + (threadIdx.x >> 6);
    if (t >= a2.M) return;
    if (local_slots(fa.topk_ids, t, a2.topk, fa.num_experts, fa.expert_offset) != 0) return;
    uint4* row = reinterpret_cast<uint4*>(fa.out + t * a2.N);
    for (int i = threadIdx.x & 63; i < a2.N / 8; i += 64) row[i] = uint4{0u, 0u, 0u, 0u};
  }
}

// Stage two for a short reduction (K = I = 128 KS, KS <= 5) at decode block
// sizes (16 NCG routes): the tile of run_tile with one wave per 64-row group
// (4 row groups, 256 output columns per workgroup, every K step), except
// that (1) the block's intermediate rows, the B operand all four waves
// share, are loaded once per workgroup into LDS (piece p of token t's 128-byte
// step row in slot p ^ ((t >> 1) & 7), so the 16 lanes of one operand read
// hit distinct bank slots) instead of once per wave, and (2) each wave issues
// the weight fragments of all KS steps before its first MFMA: KS x 4 KB in
// flight per wave, one memory latency per tile instead of one per prefetch
// window.  Same MFMA sequence per output, so the same result bit for bit.
template <int NCG, int KS>
__global__ void __launch_bounds__(256) short_k_kernel(GemmArgs args) {
  constexpr int BM = 16 * NCG;
  constexpr int PIECES = KS * BM * 8;            // 16-byte pieces of the block's B rows
  __shared__ __attribute__((aligned(16))) uint8_t sB[PIECES * 16];   // [step][token][slot]
  __shared__ __attribute__((aligned(16))) uint32_t sBs[BM * KS];      // token scales [token][step]
  __shared__ __attribute__((aligned(16))) uint8_t scr_all[4][kStage2Scratch];
  const int N = args.N, M = args.M;
  constexpr int K = KS * 128;
  const int NG = N / 256;
  const int nblk = *args.num_padded / BM;
  const int T = nblk * NG;
  if ((int)blockIdx.x >= T) return;
  const int tile = xcd_tile(blockIdx.x, T);
  const int b = tile / NG, wgg = tile - b * NG;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = wgg * 4 + wave;
  const int t16 = lane & 15, g = lane >> 4;
  const int32_t* ids = args.sorted_ids + (int64_t)b * BM;

  int rid[NCG];
  int nact = 0;
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    rid[c] = ids[c * 16 + t16];
    if (__ballot(rid[c] != M) != 0) nact = c + 1;
  }
  const int e = args.block_expert[b];

  // B rows of the block (sorted positions b BM .. + BM, contiguous in the
  // intermediate) and their scale words, into registers first
  constexpr int PER_THREAD = (PIECES + 255) / 256;
  v4i piece[PER_THREAD];
  const uint8_t* brows = args.bq + (int64_t)b * BM * K;
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int q = (int)threadIdx.x + 256 * i;     // LDS piece q = (s BM + t) 8 + slot
    if (q < PIECES) {
      const int slot = q & 7, t = (q >> 3) % BM, st = (q >> 3) / BM;
      const int p = slot ^ ((t >> 1) & 7);
      piece[i] = *reinterpret_cast<const v4i*>(brows + (int64_t)t * K + st * 128 + p * 16);
    }
  }
  uint32_t sword = 0;
  if ((int)threadIdx.x < BM * KS) {
    const int t = threadIdx.x / KS, st = threadIdx.x - t * KS;
    sword = *reinterpret_cast<const uint32_t*>(args.bs + ((int64_t)b * BM + t) * (K / 32) + 4 * st);
  }

  // every K step's weight fragments of this wave's 64 rows
  const uint8_t* wp = args.w + (int64_t)e * ((int64_t)N * K / 2) + (int64_t)grp * KS * 4096 + lane * 16;
  const uint8_t* wsp = args.ws + (int64_t)e * ((int64_t)N * K / 32) + (int64_t)grp * KS * 256 + lane * 4;
  v4i a[KS][4];
  uint32_t sa[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
#pragma unroll
    for (int t = 0; t < 4; ++t) a[st][t] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + st * 4096 + t * 1024));
    sa[st] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsp + st * 256));
  }

  // the routes' slots and routing weights, for the epilogue
  int64_t slot[NCG];
  float wt[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    const bool v = rid[c] != M;
    slot[c] = v ? route_slot(rid[c], args.topk) : -1;
    wt[c] = v ? args.topk_weights[slot[c]] : 0.f;
  }

#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int q = (int)threadIdx.x + 256 * i;
    if (q < PIECES) *reinterpret_cast<v4i*>(sB + q * 16) = piece[i];
  }
  if ((int)threadIdx.x < BM * KS) sBs[threadIdx.x] = sword;
  // the LDS writes of every wave are done (the barrier alone does not wait
  // for the weight loads still in flight)
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0) only
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");

  v4f acc[4][NCG];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < NCG; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < KS; ++st) {
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      if (c < nact) {
        const int tok = c * 16 + t16;
        const int sw = (tok >> 1) & 7;
        const uint8_t* row = sB + (st * BM + tok) * 128;
        const v8i bb = join8(*reinterpret_cast<const v4i*>(row + ((g ^ sw) << 4)),
                             *reinterpret_cast<const v4i*>(row + (((4 + g) ^ sw) << 4)));
        const uint32_t sb = (sBs[tok * KS + st] >> (8 * g)) & 0xFFu;
        acc[0][c] = mfma_fp4_fp8<0>(a[st][0], bb, acc[0][c], sa[st], sb);
        acc[1][c] = mfma_fp4_fp8<1>(a[st][1], bb, acc[1][c], sa[st], sb);
        acc[2][c] = mfma_fp4_fp8<2>(a[st][2], bb, acc[2][c], sa[st], sb);
        acc[3][c] = mfma_fp4_fp8<3>(a[st][3], bb, acc[3][c], sa[st], sb);
      }
    }
  }

  uint8_t* scr = &scr_all[wave][0];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    if (c < nact) {
      const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
      stage2_store(part, slot[c], wt[c], args, grp, g, scr);
    }
  }
}

template <int NCG, int KS>
hipError_t launch_short_k(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  const int64_t grid = max_blocks * (a.N / 256);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((short_k_kernel<NCG, KS>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int NCG>
hipError_t launch_stage2_short(const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  switch (a.K / 128) {
    case 1: return launch_short_k<NCG, 1>(a, max_blocks, stream);
    case 2: return launch_short_k<NCG, 2>(a, max_blocks, stream);
    case 3: return launch_short_k<NCG, 3>(a, max_blocks, stream);
    case 4: return launch_short_k<NCG, 4>(a, max_blocks, stream);
    default: return launch_short_k<NCG, 5>(a, max_blocks, stream);
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

template <int NCG, int NWK2, int PD1, int PD2>
hipError_t launch_fused_t(const GemmArgs& a1, const GemmArgs& a2, FusedArgs fa, int64_t max_blocks,
                          hipStream_t stream) {
  const int64_t ng1 = a1.N / 64, ng2 = a2.N / ((4 / NWK2) * 64);
  const int64_t g1 = (max_blocks * ng1 + 7) / 8 * 8, g2 = (max_blocks * ng2 + 7) / 8 * 8;
  const int64_t g3 = ((int64_t)a2.M + 3) / 4;
  if (g1 + g2 + g3 <= 0) return hipSuccess;
  fa.ng1 = (int)ng1;
  fa.g1 = (int)g1;
  fa.g2 = (int)g2;
  hipLaunchKernelGGL((fused_kernel<NCG, NWK2, PD1, PD2>), dim3((unsigned)(g1 + g2 + g3)), dim3(256), 0,
                     stream, a1, a2, fa);
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
  const bool short_k = a.K <= 640 && a.N % 256 == 0;   // K is a multiple of 128
  switch (a.bm) {
    case 16:
      if (short_k) return launch_stage2_short<1>(a, max_blocks, stream);
      return a.K >= 1024 ? launch_gemm<2, 1, 4, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream)
                         : launch_gemm<2, 1, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 32:
      if (short_k) return launch_stage2_short<2>(a, max_blocks, stream);
      return launch_gemm<2, 2, 1, MOE_S2_PD, MOE_NT_SMALL>(a, max_blocks, stream);
    case 64:
    case 128: return launch_tile(2, a, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

// The fused decode launch for blocks of 16 or 32 routes, with the kernel
// shapes of the separate stage launches above.
hipError_t launch_fused(const GemmArgs& a1, const GemmArgs& a2, const FusedArgs& fa, int64_t max_blocks,
                        hipStream_t stream) {
  switch (a1.bm) {
    case 16:
      return a2.K >= 1024 ? launch_fused_t<1, 4, MOE_S1_PD, MOE_S2_PD>(a1, a2, fa, max_blocks, stream)
                          : launch_fused_t<1, 1, MOE_S1_PD, MOE_S2_PD>(a1, a2, fa, max_blocks, stream);
    case 32: return launch_fused_t<2, 1, MOE_S1_PD, MOE_S2_PD>(a1, a2, fa, max_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
