// Grouped GEMMs of the A8W4 MoE layer for blocks of 64 or 128 routes, where an
// expert's rows are many enough that the MFMAs, not the weight stream, bound
// the time.  Same computation and epilogues as gemm.hip (stage one: SiLU(gate)
// * up and per-1x32 FP8 requantisation of the intermediate; stage two: routing
// weight and per-route rows; aiter PR 5609, "Add DeepSeek V4.1 Flash TP4
// gfx950 MoE tuning", Configuration), organised for operand reuse:
//
//   workgroup tile  256 weight rows x BM tokens (BM = 32 CGW)
//   waves           8 compute waves as 4 x 2: wave (wr, wc) computes rows
//                   [64 wr, +64) (one 64-row group, 4 MFMA tiles) x tokens
//                   [wc BM/2, +BM/2); and 4 loader waves that only move data.
//                   Each SIMD runs two compute waves (one hides the other's
//                   LDS reads and barrier waits) and one loader (a loader
//                   stalled on the memory pipeline never holds back MFMAs).
//   K step          128: 16 KB of packed weights, BM x 128 B of token codes,
//                   1 KB of weight scales and BM x 4 B of token scales
//   staging         a ring of S such steps in LDS, filled by direct
//                   global-to-LDS loads (no registers involved): while the
//                   MFMAs consume step s, steps s + 1 .. s + S - 1 are in
//                   flight; one workgroup barrier per step.
//
// LDS layout of one step (offsets in bytes):
//   A   [4 row groups][4 tiles][64 lanes][16]   the packed chunk as stored
//   B   [BM tokens][8 slots of 16]              piece p of token t sits in slot
//                                               p ^ ((t >> 1) & 7), so the 16
//                                               lanes of one operand read hit 16
//                                               distinct 16-byte bank slots
//   As  [4 row groups][64 lanes][4]             E8M0 weight scales
//   Bs  [BM tokens][4]                          E8M0 token scales, used only
//                                               when the tile's scales do not
//                                               fit the preload area below;
//                                               loader l < BM/64 loads tokens
//                                               64 l + lane
//
// Token scales otherwise: all BM x K/32 of the tile in a separate LDS area,
// token-major, loaded before step 0 (one short row per token instead of a
// 4-byte gather from every token row at every step).
//
// Barrier s: every loader has waited until its loads of step s have landed
// (vmcnt), every compute wave until its LDS reads of step s - 1 are done.  It
// publishes step s and frees the slot of step s - 1, which the loaders refill
// with step s + S - 1 while the compute waves work on step s.
#include "gemm_common.hpp"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;

// M0 carries the LDS base of the direct loads below; no other code of this
// kernel uses M0 (clang warns about naming a reserved register as clobbered).
#pragma clang diagnostic ignored "-Winline-asm"

// Direct global-to-LDS loads: lane l's 16 (or 4) bytes at g go to LDS byte
// lds + 16 l (or 4 l); lds must be the same in every lane.  Written as inline
// assembly so that the compiler, which cannot tell the ring's slots apart,
// does not wait for every load in flight before each LDS read; the kernel
// waits for them itself (vmcnt) before the barrier that publishes a slot.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
// The same with the non-temporal hint, for weights that stage two streams
// past the caches (each 256-row slice of an expert is read by the few blocks
// of that expert, side by side; measured faster than cached loads for every
// prefill stage-two shape, e.g. prefill-shared 4096 tokens 274 -> 251 us,
// local slice 16384 tokens 383 -> 361 us).
__device__ __forceinline__ void dma16nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
template <int STAGE>
__device__ __forceinline__ void dma16w(const void* g, uint32_t lds) {
  if constexpr (STAGE == 2) dma16nt(g, lds);
  else dma16(g, lds);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)p);
}

template <int CGW>
struct TileGeom {
  static constexpr int BM = 32 * CGW;               // tokens
  static constexpr int NBCH = CGW;                  // 1 KB token chunks per loader and step
  static constexpr int A = 0;
  static constexpr int B = A + 16384;
  static constexpr int AS = B + BM * 128;
  static constexpr int BS = AS + 1024;
  static constexpr int BYTES = BS + 1024;
  static constexpr int NBS = BM / 64;               // loaders that also load token scales
  static constexpr int LOADS = 4 + NBCH + 1;        // per loader and step: A, B chunks, As (+ Bs)
};

// s_waitcnt immediates (gfx9 encoding): wait on the vector-memory counter
// only, or on the LDS/scalar counter only.
constexpr int vmcnt_only(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int lgkmcnt_zero() { return 15 | (3 << 14) | (7 << 4); }

// A workgroup barrier without the memory fences of __syncthreads (those would
// also wait for every direct-to-LDS load still in flight).
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile order.  In block-major order (t = b NT + wgt) the tiles of one expert
// form the run [f NT, (f + nb) NT), f its first block and nb its block count.
// Inside that run the tiles are taken slice-major (wgt = l / nb, b = f + l % nb)
// so that the nb blocks that read the same weight slice run side by
// side on one XCD and share it through its L2, while the expert's token
// blocks stay resident there across the slices.  f and nb come from the run
// of equal entries of block_expert around block t / NT (every wave finds
// them itself with two 64-wide ballots; block_expert is sorted).
__device__ __forceinline__ void expert_major(int t, int NT, int nblk, const int32_t* __restrict__ block_expert,
                                             int& b, int& wgt) {
  const int lane = threadIdx.x & 63;
  const int b0 = t / NT;
  const int e = block_expert[b0];
  int back = 0;   // blocks of e at or before b0
  for (;;) {
    const int idx = b0 - back - lane;
    const bool eq = idx >= 0 && block_expert[idx] == e;
    const unsigned long long m = __ballot(eq);
    const int run = (~m == 0ull) ? 64 : __builtin_ctzll(~m);
    back += run;
    if (run < 64) break;
  }
  int fwd = 0;    // blocks of e after b0
  for (;;) {
    const int idx = b0 + 1 + fwd + lane;
    const bool eq = idx < nblk && block_expert[idx] == e;
    const unsigned long long m = __ballot(eq);
    const int run = (~m == 0ull) ? 64 : __builtin_ctzll(~m);
    fwd += run;
    if (run < 64) break;
  }
  const int f = b0 - back + 1, nb = back + fwd;
  const int l = t - f * NT;
  wgt = l / nb;
  b = f + (l - wgt * nb);
}

constexpr int kComputeWaves = 8, kLoaderWaves = 4;
// LDS for a tile's token scales, loaded once at the tile's start (a gather of
// one short row per token) instead of one 4-byte gather per token and step:
// up to block_m x K / 32 bytes (K <= 8192 at block_m 128), so that a loader
// issues at most 32 such loads.
constexpr int kScalePreloadBytes = 32 * 1024;

// PRE: the tile's token scales are preloaded (BM x K/32 <= kScalePreloadBytes).
// SC4 (without PRE): token scales come four steps at a time, one 16-byte load
// per token every fourth step into a double-buffered area, instead of a
// 4-byte gather per token and step (a quarter of those L2 requests); needs
// K/128 a multiple of 4 (stage one: K = H, a multiple of 512) and 16-byte
// aligned scale rows.
template <int STAGE, int CGW, int S, bool PRE, bool SC4 = false>
__global__ void __launch_bounds__(64 * (kComputeWaves + kLoaderWaves), 3) tile_kernel(GemmArgs args) {
  using G = TileGeom<CGW>;
  constexpr int BM = G::BM;
  static_assert(!(PRE && SC4), "one way of loading token scales");
  static_assert(!SC4 || S <= 5, "a scale buffer is refilled once its four steps are read");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S][G::BYTES];
  // all token scales of the tile, [BM tokens][K / 32], when they fit
  __shared__ __attribute__((aligned(16))) uint8_t spre[PRE ? kScalePreloadBytes : 16];
  // SC4: [2 buffers][BM tokens][4 steps][4 scale bytes]; buffer q & 1 holds
  // steps 4q .. 4q + 3
  __shared__ __attribute__((aligned(16))) uint8_t ssc[SC4 ? 2 * BM * 16 : 16];

  const int N = args.N, K = args.K, M = args.M;
  const int KS = K / 128;
  const int NT = N / 256;
  const int nblk = *args.num_padded / BM;
  const int T = nblk * NT;
  if ((int)blockIdx.x >= T) return;
  int b, wgt;
  expert_major(xcd_tile(blockIdx.x, T), NT, nblk, args.block_expert, b, wgt);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases go to M0
  const int32_t* ids = args.sorted_ids + (int64_t)b * BM;

  if (wave >= kComputeWaves) {
    // ------------------------------------------------------------ loader
    const int l = wave - kComputeWaves;
    const int e = args.block_expert[b];
    const int first = ids[0];   // a block always starts with a route
    // B row of block token t; padding tokens read a real row (their
    // columns are never stored, the load only has to stay in bounds)
    auto brow = [&](int t) -> int64_t {
      if (STAGE == 1) {
        const int r = ids[t];
        return (int64_t)((r == M ? first : r) & 0xFFFFFF);
      }
      return (int64_t)b * BM + t;
    };
    const uint8_t* gA = args.w + (int64_t)e * ((int64_t)N * K / 2) +
                        (int64_t)(wgt * 4 + l) * KS * 4096 + lane * 16;
    const uint8_t* gAs = args.ws + (int64_t)e * ((int64_t)N * K / 32) +
                         (int64_t)(wgt * 4 + l) * KS * 256 + lane * 4;
    const uint8_t* gB[G::NBCH];
#pragma unroll
    for (int i = 0; i < G::NBCH; ++i) {
      const int t = 8 * (l * G::NBCH + i) + (lane >> 3);
      const int piece = (lane & 7) ^ ((t >> 1) & 7);
      gB[i] = args.bq + brow(t) * K + piece * 16;
    }
    constexpr int NBS = G::NBS;
    // per-step token scales (only without the preload): loader l < NBS
    // brings those of tokens [64 l, +64)
    const bool has_bs = !PRE && l < NBS;
    const uint8_t* gBs = args.bs + brow((l % NBS) * 64 + lane) * (K / 32);
    const uint32_t lds0 = lds_addr(&smem[0][0]);
    if constexpr (PRE) {
      // the tile's token scales as one flat run of BM * KS words (word d:
      // token d / KS, step d % KS), 64 words per load, the loaders taking
      // turns; issued before step 0, so barrier 0 also covers them
      const uint32_t pre0 = lds_addr(&spre[0]);
      // the rows of tokens lane and 64 + lane, fetched once; each load then
      // takes its tokens' rows from the lanes that hold them
      const int row_lo = (int)brow(lane);
      const int row_hi = BM > 64 ? (int)brow(64 + lane) : 0;
      for (int d0 = l * 64; d0 < BM * KS; d0 += kLoaderWaves * 64) {
        const int d = d0 + lane;
        const int u = d / KS;
        const int r_lo = __shfl(row_lo, u & 63), r_hi = __shfl(row_hi, u & 63);
        const int64_t row = u < 64 ? r_lo : r_hi;
        dma4(args.bs + row * (K / 32) + 4 * (d - u * KS), pre0 + (uint32_t)d0 * 4);
      }
    }
    // A block's routes come first and its padding last, so when the first
    // token of this loader's chunks is padding all of them are: their rows
    // feed only output columns that are never stored, and their loads are
    // skipped (a block of 128 routes holding 64 reads half the token bytes).
    const bool skip_tok = ids[8 * l * G::NBCH] == M;
    auto run_loader = [&](auto skip_tag) {
      constexpr bool SKIP = decltype(skip_tag)::value;
      constexpr int LOADS = G::LOADS - (SKIP ? G::NBCH : 0);
      auto issue = [&](int s) {
        const uint32_t base = lds0 + (uint32_t)(s % S) * G::BYTES;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          dma16w<STAGE>(gA + (int64_t)s * 4096 + t * 1024, base + G::A + l * 4096 + t * 1024);
        if constexpr (!SKIP) {
#pragma unroll
          for (int i = 0; i < G::NBCH; ++i) dma16(gB[i] + s * 128, base + G::B + (l * G::NBCH + i) * 1024);
        }
        dma4(gAs + (int64_t)s * 256, base + G::AS + l * 256);
        if (has_bs) {
          if constexpr (SC4) {
            if ((s & 3) == 0) dma16(gBs + 4 * s, lds_addr(&ssc[0]) + (uint32_t)((s >> 2) & 1) * (BM * 16) + l * 1024);
          } else {
            dma4(gBs + 4 * s, base + G::BS + l * 256);
          }
        }
      };
#pragma unroll
      for (int s = 0; s < S - 1; ++s)
        if (s < KS) issue(s);
      for (int s = 0; s < KS; ++s) {
        // barrier s publishes step s: it has landed once at most the loads of
        // steps s+1 .. s+S-2 are outstanding (near the end: none)
        if (s + S - 2 < KS) {
          if (has_bs) {
            if constexpr (SC4) {
              // steps s+1 .. s+S-2 (at most 3 of them) hold at most one
              // scale load, the one of a step that is a multiple of 4
              bool sc = false;
#pragma unroll
              for (int j = 1; j <= S - 2; ++j) sc = sc || ((s + j) & 3) == 0;
              if (sc) __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * LOADS + 1));
              else __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * LOADS));
            } else {
              __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * (LOADS + 1)));
            }
          } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * LOADS));
          }
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        }
        barrier_only();
        // every compute wave has finished reading step s - 1: refill its slot
        if (s + S - 1 < KS) issue(s + S - 1);
      }
    };
    if (skip_tok) run_loader(std::true_type{});
    else run_loader(std::false_type{});
    return;
  }

  // -------------------------------------------------------------- compute
  const int wr = wave >> 1, wc = wave & 1;
  const int t16 = lane & 15, g = lane >> 4;

  // the K loop and epilogue for NA active 16-token column groups of this
  // wave (columns past the block's last route are skipped); every compute
  // wave takes every barrier whatever its NA
  auto run = [&](auto na_tag) {
    constexpr int NA = decltype(na_tag)::value;
    // stage two: slots and routing weights of this wave's columns, fetched
    // before the K loop so the epilogue does not wait for them
    int64_t slot[NA > 0 ? NA : 1];
    float wt[NA > 0 ? NA : 1];
    if constexpr (STAGE == 2) {
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        const int rid = ids[wc * CGW * 16 + c * 16 + t16];
        slot[c] = rid == M ? -1 : route_slot(rid, args.topk);
        wt[c] = rid == M ? 0.f : args.topk_weights[slot[c]];
      }
    }
    v4f acc[4][NA > 0 ? NA : 1];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < NA; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

    if constexpr (NA == 0) {
      // no columns: only the barriers (0 .. KS - 1)
      for (int s = 0; s < KS; ++s) barrier_only();
    } else {
      // Operands are read from LDS one column group ahead of the MFMAs that
      // use them, and the next step's weight fragments and first column group
      // right after the barrier that publishes that step, while the last
      // column group's MFMAs of the current step still run: the MFMA pipe is
      // not left idle across the barrier.  Two register sets of weight
      // fragments (cur / nxt) and two of token fragments (bb[0], bb[1]).
      struct AOps {
        v4i a[4];
        uint32_t sa;
      };
      v8i bb[2];
      uint32_t sb[2];
      auto read_a = [&](AOps& o, int s) {
        const uint8_t* base = smem[s % S];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o.a[t] = *reinterpret_cast<const v4i*>(base + G::A + wr * 4096 + t * 1024 + lane * 16);
        o.sa = *reinterpret_cast<const uint32_t*>(base + G::AS + wr * 256 + lane * 4);
      };
      auto read_b = [&](int i, int s, int c) {
        const uint8_t* base = smem[s % S];
        const int tok = wc * CGW * 16 + c * 16 + t16;
        const int sw = (tok >> 1) & 7;
        const uint8_t* row = base + G::B + tok * 128;
        bb[i] = join8(*reinterpret_cast<const v4i*>(row + ((g ^ sw) << 4)),
                      *reinterpret_cast<const v4i*>(row + (((4 + g) ^ sw) << 4)));
        sb[i] = PRE ? spre[(tok * KS + s) * 4 + g]
                    : SC4 ? ssc[((s >> 2) & 1) * (BM * 16) + tok * 16 + (s & 3) * 4 + g]
                          : base[G::BS + tok * 4 + g];
      };
      // step s with its weight fragments in cur and its first column group
      // in bb[P]; when NEXT (s + 1 < KS) also takes barrier s + 1 and reads
      // step s + 1's into nxt and bb[(P + NA) % 2]
      auto step = [&](auto p_tag, auto next_tag, int s, AOps& cur, AOps& nxt) {
        constexpr int P = decltype(p_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
#pragma unroll
        for (int c = 0; c < NA; ++c) {
          const int i = (P + c) % 2;
          // scheduling fences: the reads are issued before this group's
          // MFMAs (so they overlap them), and no read moves to another group
          // (hoisting reads of later groups runs out of registers)
          __builtin_amdgcn_sched_barrier(0);
          if (c + 1 < NA) {
            read_b((P + c + 1) % 2, s, c + 1);
          } else if (NEXT) {
            // every read of step s has landed: barrier s + 1 frees its slot
            // and publishes step s + 1
            __builtin_amdgcn_s_waitcnt(lgkmcnt_zero());
            barrier_only();
            read_a(nxt, s + 1);
            read_b((P + NA) % 2, s + 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          acc[0][c] = mfma_fp4_fp8<0>(cur.a[0], bb[i], acc[0][c], cur.sa, sb[i]);
          acc[1][c] = mfma_fp4_fp8<1>(cur.a[1], bb[i], acc[1][c], cur.sa, sb[i]);
          acc[2][c] = mfma_fp4_fp8<2>(cur.a[2], bb[i], acc[2][c], cur.sa, sb[i]);
          acc[3][c] = mfma_fp4_fp8<3>(cur.a[3], bb[i], acc[3][c], cur.sa, sb[i]);
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using IQ = std::integral_constant<int, NA % 2>;   // bb index of odd steps' first group
      using Yes = std::true_type;
      using No = std::false_type;
      AOps o0, o1;
      barrier_only();   // barrier 0 publishes step 0
      read_a(o0, 0);
      read_b(0, 0, 0);
      int s = 0;
      for (; s + 2 < KS; s += 2) {
        step(I0{}, Yes{}, s, o0, o1);
        step(IQ{}, Yes{}, s + 1, o1, o0);
      }
      if (s + 1 < KS) {
        step(I0{}, Yes{}, s, o0, o1);
        step(IQ{}, No{}, s + 1, o1, o0);
      } else {
        step(I0{}, No{}, s, o0, o1);
      }
    }

    const int grp = wgt * 4 + wr;
    if constexpr (STAGE == 1) {
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        const int col = wc * CGW * 16 + c * 16 + t16;
        stage1_store(part, (int64_t)b * BM + col, grp, N / 2, g, args.out_q, args.out_s);
      }
    } else {
      // the route rows go out through LDS scratch: a wave-private area in
      // one of the two ring slots no wave touches after the last barrier
      // (the slots of steps KS - 3 and KS - 2, or unused ones)
      uint8_t* scr = smem[(KS + (wave >> 2)) % S] + (wave & 3) * kStage2Scratch;
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage2_store(part, slot[c], wt[c], args, grp, g, scr);
      }
    }
  };

  int nact = 0;
#pragma unroll
  for (int c = 0; c < CGW; ++c)
    if (__ballot(ids[wc * CGW * 16 + c * 16 + t16] != M) != 0) nact = c + 1;
  nact = __builtin_amdgcn_readfirstlane(nact);
  if (nact == CGW) run(std::integral_constant<int, CGW>{});
  else if (nact == 0) run(std::integral_constant<int, 0>{});
  else if (nact == 1) run(std::integral_constant<int, 1>{});
  else if constexpr (CGW > 2) {
    if (nact == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
  }
}

// ------------------------------------------------ short K: tokens resident
//
// For a short reduction (K <= kResidentBytes / BM, e.g. stage two at I 640)
// a 256-row tile has only a few K steps, so the pipeline fill and the
// epilogue dominate and every slice re-reads the block's tokens.  Here a
// workgroup keeps the block's whole token tile (BM x K codes and their
// scales) in LDS, loaded once, and runs NS consecutive 256-row weight slices
// against it: NS x KS steps in which only the weights stream through the
// ring, an epilogue after every KS of them.  Same waves and per-step MFMAs as
// tile_kernel; the loaders run on into the next slice while the compute
// waves store the previous one.
constexpr int kResidentBytes = 80 * 1024;

template <int STAGE, int CGW, int S, int NS>
__global__ void __launch_bounds__(64 * (kComputeWaves + kLoaderWaves), 3) tile_resident_kernel(GemmArgs args) {
  constexpr int BM = 32 * CGW;
  constexpr int NBCH = CGW;                 // 1 KB token chunks per loader and K step
  constexpr int SLOT = 16384 + 1024;        // ring slot: A [4][4][64][16], As [4][64][4]
  constexpr int LOADS = 4 + 1;              // per loader and step
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S][SLOT];
  // token codes, step-major: step s at s * BM * 128, laid out as tile_kernel's B
  __shared__ __attribute__((aligned(1024))) uint8_t sB[kResidentBytes];
  // token scales, token-major [BM][K / 32]
  __shared__ __attribute__((aligned(16))) uint8_t sBs[kResidentBytes / 32];
  // stage two: wave-private scratch of the route-row stores (the ring holds
  // the next slice's steps while a slice is stored)
  __shared__ __attribute__((aligned(16))) uint8_t scr_all[STAGE == 2 ? kComputeWaves : 1]
                                                        [STAGE == 2 ? kStage2Scratch : 16];

  const int N = args.N, K = args.K, M = args.M;
  const int KS = K / 128;
  const int NG = N / (256 * NS);            // slice groups per block
  const int nblk = *args.num_padded / BM;
  const int T = nblk * NG;
  if ((int)blockIdx.x >= T) return;
  int b, sg;
  expert_major(xcd_tile(blockIdx.x, T), NG, nblk, args.block_expert, b, sg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* ids = args.sorted_ids + (int64_t)b * BM;
  const int Q = NS * KS;                    // steps of the tile: slice q / KS, K step q % KS

  if (wave >= kComputeWaves) {
    // ------------------------------------------------------------ loader
    const int l = wave - kComputeWaves;
    const int e = args.block_expert[b];
    const int first = ids[0];
    auto brow = [&](int t) -> int64_t {
      if (STAGE == 1) {
        const int r = ids[t];
        return (int64_t)((r == M ? first : r) & 0xFFFFFF);
      }
      return (int64_t)b * BM + t;
    };
    // the resident token tile: loader l brings chunks l NBCH .. of every step
#pragma unroll
    for (int i = 0; i < NBCH; ++i) {
      const int t = 8 * (l * NBCH + i) + (lane >> 3);
      const int piece = (lane & 7) ^ ((t >> 1) & 7);
      const uint8_t* src = args.bq + brow(t) * K + piece * 16;
      const uint32_t dst = lds_addr(&sB[0]) + (uint32_t)(l * NBCH + i) * 1024;
      for (int ks = 0; ks < KS; ++ks) dma16(src + ks * 128, dst + (uint32_t)ks * BM * 128);
    }
    {
      // token scales as one flat run of BM * KS words (word d: token d / KS,
      // step d % KS), each load taking its tokens' rows from the lanes that
      // hold them
      const int row_lo = (int)brow(lane);
      const int row_hi = BM > 64 ? (int)brow(64 + lane) : 0;
      const uint32_t s0 = lds_addr(&sBs[0]);
      for (int d0 = l * 64; d0 < BM * KS; d0 += kLoaderWaves * 64) {
        const int d = d0 + lane;
        const int u = d / KS;
        const int r_lo = __shfl(row_lo, u & 63), r_hi = __shfl(row_hi, u & 63);
        const int64_t row = u < 64 ? r_lo : r_hi;
        dma4(args.bs + row * (K / 32) + 4 * (d - u * KS), s0 + (uint32_t)d0 * 4);
      }
    }
    // weights: slice j of the group is row groups (sg NS + j) 4 + l of expert e
    const uint8_t* gA = args.w + (int64_t)e * ((int64_t)N * K / 2) + (int64_t)(sg * NS * 4 + l) * KS * 4096 +
                        lane * 16;
    const uint8_t* gAs = args.ws + (int64_t)e * ((int64_t)N * K / 32) + (int64_t)(sg * NS * 4 + l) * KS * 256 +
                         lane * 4;
    const uint32_t lds0 = lds_addr(&ring[0][0]);
    auto issue = [&](int q) {
      const int j = q / KS, ks = q - j * KS;
      const int64_t step = (int64_t)j * 4 * KS + ks;   // row group advances by 4 per slice
      const uint32_t base = lds0 + (uint32_t)(q % S) * SLOT;
#pragma unroll
      for (int t = 0; t < 4; ++t) dma16w<STAGE>(gA + step * 4096 + t * 1024, base + l * 4096 + t * 1024);
      dma4(gAs + step * 256, base + 16384 + l * 256);
    };
#pragma unroll
    for (int q = 0; q < S - 1; ++q)
      if (q < Q) issue(q);
    for (int q = 0; q < Q; ++q) {
      // barrier q publishes step q (and, at q = 0, the resident tile issued
      // before it)
      if (q + S - 2 < Q) __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * LOADS));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      barrier_only();
      if (q + S - 1 < Q) issue(q + S - 1);
    }
    return;
  }

  // -------------------------------------------------------------- compute
  const int wr = wave >> 1, wc = wave & 1;
  const int t16 = lane & 15, g = lane >> 4;
  uint8_t* scr = &scr_all[STAGE == 2 ? wave : 0][0];

  auto run = [&](auto na_tag) {
    constexpr int NA = decltype(na_tag)::value;
    int64_t slot[NA > 0 ? NA : 1];
    float wt[NA > 0 ? NA : 1];
    if constexpr (STAGE == 2) {
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        const int rid = ids[wc * CGW * 16 + c * 16 + t16];
        slot[c] = rid == M ? -1 : route_slot(rid, args.topk);
        wt[c] = rid == M ? 0.f : args.topk_weights[slot[c]];
      }
    }
    // the store lanes' route slots, the same for every slice
    int sl2[NA > 0 ? NA : 1][2];
    if constexpr (STAGE == 2) {
#pragma unroll
      for (int c = 0; c < NA; ++c) stage2_store_slots(slot[c], sl2[c]);
    }
    for (int j = 0; j < NS; ++j) {
      v4f acc[4][NA > 0 ? NA : 1];
      // K step ks of slice j; the first step of a slice starts its
      // accumulators from a literal zero (no per-slice register clearing)
      auto kstep = [&](int ks, auto first_tag) {
        constexpr bool FIRST = decltype(first_tag)::value;
        const int q = j * KS + ks;
        __builtin_amdgcn_s_waitcnt(lgkmcnt_zero());
        barrier_only();
        if constexpr (NA > 0) {
          const uint8_t* base = ring[q % S];
          v4i a[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            a[t] = *reinterpret_cast<const v4i*>(base + wr * 4096 + t * 1024 + lane * 16);
          const uint32_t sa = *reinterpret_cast<const uint32_t*>(base + 16384 + wr * 256 + lane * 4);
          const uint8_t* bstep = sB + ks * BM * 128;
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NA; ++c) {
            const int tok = wc * CGW * 16 + c * 16 + t16;
            const int sw = (tok >> 1) & 7;
            const uint8_t* row = bstep + tok * 128;
            const v8i bb = join8(*reinterpret_cast<const v4i*>(row + ((g ^ sw) << 4)),
                                 *reinterpret_cast<const v4i*>(row + (((4 + g) ^ sw) << 4)));
            const uint32_t sb = sBs[(tok * KS + ks) * 4 + g];
            acc[0][c] = mfma_fp4_fp8<0>(a[0], bb, FIRST ? zero : acc[0][c], sa, sb);
            acc[1][c] = mfma_fp4_fp8<1>(a[1], bb, FIRST ? zero : acc[1][c], sa, sb);
            acc[2][c] = mfma_fp4_fp8<2>(a[2], bb, FIRST ? zero : acc[2][c], sa, sb);
            acc[3][c] = mfma_fp4_fp8<3>(a[3], bb, FIRST ? zero : acc[3][c], sa, sb);
          }
        }
      };
      kstep(0, std::true_type{});
      for (int ks = 1; ks < KS; ++ks) kstep(ks, std::false_type{});
      const int grp = (sg * NS + j) * 4 + wr;
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        if constexpr (STAGE == 1) {
          const int col = wc * CGW * 16 + c * 16 + t16;
          stage1_store(part, (int64_t)b * BM + col, grp, N / 2, g, args.out_q, args.out_s);
        } else {
          stage2_store(part, slot[c], sl2[c], wt[c], args, grp, g, scr);
        }
      }
    }
  };

  int nact = 0;
#pragma unroll
  for (int c = 0; c < CGW; ++c)
    if (__ballot(ids[wc * CGW * 16 + c * 16 + t16] != M) != 0) nact = c + 1;
  nact = __builtin_amdgcn_readfirstlane(nact);
  if (nact == CGW) run(std::integral_constant<int, CGW>{});
  else if (nact == 0) run(std::integral_constant<int, 0>{});
  else if (nact == 1) run(std::integral_constant<int, 1>{});
  else if constexpr (CGW > 2) {
    if (nact == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
  }
}

#ifndef MOE_TILE_STAGES
#define MOE_TILE_STAGES 3
#endif
static_assert(MOE_TILE_STAGES >= 3, "the stage-two epilogue borrows the two ring slots not read last");

// Slices per workgroup of the token-resident kernel for this launch (0: not
// used): the token tile must fit; of the group sizes that split the 256-row
// slices evenly, the largest that still leaves eight workgroups per CU for the
// routing-free bound on the tiles (max_tiles), else the smallest.  One
// workgroup fits a CU at a time, so fewer, longer workgroups leave a larger
// last round.  Measured (stage two, us): prefill-shared 2048 tokens 10 slices
// 178, 5 slices 170; 4096 tokens 229 / 210; 8192 tokens 261 / 251; 16384
// tokens keeps 10 (4 slices 749 against 690 in an earlier version, 20 slices
// 762); at the backbone geometry's 2048 and 4096 tokens, where the blocks
// fill whole rounds, 5 slices cost 2-6 us more.
int resident_slices(const GemmArgs& a, int64_t max_tiles) {
  if ((int64_t)a.bm * a.K > kResidentBytes) return 0;
  const int slices = a.N / 256;
  int pick = 0;
  for (int ns : {4, 5, 10}) {
    if (slices % ns) continue;
    if (pick == 0 || max_tiles / ns >= 2048) pick = ns;
  }
  return pick;
}

// ------------------------------------------- A16W4 variant: BF16 tokens
//
// The tile kernel above for the A16W4 variant (BF16 activations x MXFP4
// weights): the same workgroup tile (256 weight rows x BM tokens), waves
// (8 compute, 4 loaders), ring of S K steps filled by direct loads and
// expert-major tile order.  Per K step of 128: 16 KB of packed weights,
// BM x 256 B of BF16 tokens and 1 KB of weight scales; no token scales.
// A compute wave reads its 4 tiles' FP4 fragments from LDS, converts them to
// BF16 (v_cvt_scalef32_pk_bf16_fp4 with the block scale) and runs
// v_mfma_f32_16x16x32_bf16, four per tile and column group, with the K
// assignment of gemm_a16.hip (MFMA j of a step takes K 32 q + 8 j + [0, 8) in
// lane group q).  Token piece p (16 B, 8 BF16) of token t sits in slot
// p ^ (t & 15): the 16 lanes of one operand read (16 tokens, one piece) hit
// 16 distinct 16-byte bank slots.
template <int CGW>
struct TileGeomA16 {
  static constexpr int BM = 32 * CGW;               // tokens
  static constexpr int NBCH = 2 * CGW;              // 1 KB token chunks per loader and step
  static constexpr int A = 0;
  static constexpr int B = A + 16384;
  static constexpr int AS = B + BM * 256;
  static constexpr int BYTES = AS + 1024;
  static constexpr int LOADS = 4 + NBCH + 1;        // per loader and step: A, B chunks, As
};

template <int STAGE, int CGW, int S>
__global__ void __launch_bounds__(64 * (kComputeWaves + kLoaderWaves), 3) a16_tile_kernel(GemmArgs args) {
  using G = TileGeomA16<CGW>;
  constexpr int BM = G::BM;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S][G::BYTES];

  const int N = args.N, K = args.K, M = args.M;
  const int KS = K / 128;
  const int NT = N / 256;
  const int nblk = *args.num_padded / BM;
  const int T = nblk * NT;
  if ((int)blockIdx.x >= T) return;
  int b, wgt;
  expert_major(xcd_tile(blockIdx.x, T), NT, nblk, args.block_expert, b, wgt);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* ids = args.sorted_ids + (int64_t)b * BM;

  if (wave >= kComputeWaves) {
    // ------------------------------------------------------------ loader
    const int l = wave - kComputeWaves;
    const int e = args.block_expert[b];
    const int first = ids[0];
    auto brow = [&](int t) -> int64_t {
      if (STAGE == 1) {
        const int r = ids[t];
        return (int64_t)((r == M ? first : r) & 0xFFFFFF);
      }
      return (int64_t)b * BM + t;
    };
    const uint8_t* gA = args.w + (int64_t)e * ((int64_t)N * K / 2) +
                        (int64_t)(wgt * 4 + l) * KS * 4096 + lane * 16;
    const uint8_t* gAs = args.ws + (int64_t)e * ((int64_t)N * K / 32) +
                         (int64_t)(wgt * 4 + l) * KS * 256 + lane * 4;
    // chunk i of loader l: tokens 4 (l NBCH + i) + lane / 16, LDS slot
    // lane % 16 of the token, filled with the piece that belongs there
    const uint8_t* gB[G::NBCH];
#pragma unroll
    for (int i = 0; i < G::NBCH; ++i) {
      const int t = 4 * (l * G::NBCH + i) + (lane >> 4);
      const int piece = (lane & 15) ^ (t & 15);
      gB[i] = args.bq + brow(t) * K * 2 + piece * 16;
    }
    const uint32_t lds0 = lds_addr(&smem[0][0]);
    auto issue = [&](int s) {
      const uint32_t base = lds0 + (uint32_t)(s % S) * G::BYTES;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dma16w<STAGE>(gA + (int64_t)s * 4096 + t * 1024, base + G::A + l * 4096 + t * 1024);
#pragma unroll
      for (int i = 0; i < G::NBCH; ++i) dma16(gB[i] + s * 256, base + G::B + (l * G::NBCH + i) * 1024);
      dma4(gAs + (int64_t)s * 256, base + G::AS + l * 256);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < KS) issue(s);
    for (int s = 0; s < KS; ++s) {
      if (s + S - 2 < KS) __builtin_amdgcn_s_waitcnt(vmcnt_only((S - 2) * G::LOADS));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      barrier_only();
      if (s + S - 1 < KS) issue(s + S - 1);
    }
    return;
  }

  // -------------------------------------------------------------- compute
  const int wr = wave >> 1, wc = wave & 1;
  const int t16 = lane & 15, g = lane >> 4;
  int nact = 0;
#pragma unroll
  for (int c = 0; c < CGW; ++c)
    if (__ballot(ids[wc * CGW * 16 + c * 16 + t16] != M) != 0) nact = c + 1;
  nact = __builtin_amdgcn_readfirstlane(nact);

  int64_t slot[CGW];
  float wt[CGW];
#pragma unroll
  for (int c = 0; c < CGW; ++c) {
    slot[c] = -1;
    wt[c] = 0.f;
    if (STAGE == 2) {
      const int rid = ids[wc * CGW * 16 + c * 16 + t16];
      if (rid != M) {
        slot[c] = route_slot(rid, args.topk);
        wt[c] = args.topk_weights[slot[c]];
      }
    }
  }
  v4f acc[4][CGW];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < CGW; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < KS; ++s) {
    barrier_only();   // barrier s publishes step s
    if (nact > 0) {
      const uint8_t* base = smem[s % S];
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4i*>(base + G::A + wr * 4096 + t * 1024 + lane * 16);
      const uint32_t sa = *reinterpret_cast<const uint32_t*>(base + G::AS + wr * 256 + lane * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 aj[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = (uint32_t)(j == 0 ? a[t].x : j == 1 ? a[t].y : j == 2 ? a[t].z : a[t].w);
          aj[t] = fp4x8_to_bf16(w, e8m0_to_f32((sa >> (8 * t)) & 0xFFu));
        }
#pragma unroll
        for (int c = 0; c < CGW; ++c) {
          if (c < nact) {
            const int tok = wc * CGW * 16 + c * 16 + t16;
            const int slot_j = (4 * g + j) ^ (tok & 15);
            const bf16x8 bj = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4i*>(base + G::B + tok * 256 + slot_j * 16));
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aj[t], bj, acc[t][c], 0, 0, 0);
          }
        }
      }
    }
    // every LDS read of step s is done before barrier s + 1 frees its slot
    __builtin_amdgcn_s_waitcnt(lgkmcnt_zero());
  }

  const int grp = wgt * 4 + wr;
  if constexpr (STAGE == 1) {
#pragma unroll
    for (int c = 0; c < CGW; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        a16_stage1_store(part, (int64_t)b * BM + wc * CGW * 16 + c * 16 + t16, grp, N / 2, g,
                         reinterpret_cast<uint16_t*>(args.out_q));
      }
    }
  } else {
    // route rows through LDS scratch in a ring slot no wave reads after the
    // last barrier (the slots of steps KS - 3 and KS - 2, or unused ones)
    uint8_t* scr = smem[(KS + (wave >> 2)) % S] + (wave & 3) * kStage2Scratch;
#pragma unroll
    for (int c = 0; c < CGW; ++c) {
      if (c < nact) {
        const v4f part[4] = {acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        stage2_store(part, slot[c], wt[c], args, grp, g, scr);
      }
    }
  }
}

// Token-resident kernel where resident_slices allows, else tile_kernel. Its
// scale preload pays at block_m 64 (stage one at local-slice M=4096: -6 %); at
// block_m 128 the wait before step 0 costs more than the per-step gathers it
// saves (+4 % at M=16384), so those tiles keep the per-step loads.
template <int STAGE, int CGW, int S>
void launch_one(const GemmArgs& a, dim3 g, dim3 blk, hipStream_t stream) {
  const int ns = resident_slices(a, g.x);
  if (ns > 0) {
    const dim3 gr((unsigned)(g.x / ns));
    switch (ns) {
      case 4: hipLaunchKernelGGL((tile_resident_kernel<STAGE, CGW, S, 4>), gr, blk, 0, stream, a); return;
      case 5: hipLaunchKernelGGL((tile_resident_kernel<STAGE, CGW, S, 5>), gr, blk, 0, stream, a); return;
      default: hipLaunchKernelGGL((tile_resident_kernel<STAGE, CGW, S, 10>), gr, blk, 0, stream, a); return;
    }
  }
  if (CGW == 2 && 32 * CGW * (a.K / 128) * 4 <= kScalePreloadBytes)
    hipLaunchKernelGGL((tile_kernel<STAGE, CGW, S, true>), g, blk, 0, stream, a);
  else if (STAGE == 1 && (a.K / 128) % 4 == 0 && ((uintptr_t)a.bs & 15) == 0)
    hipLaunchKernelGGL((tile_kernel<STAGE, CGW, S, false, true>), g, blk, 0, stream, a);
  else
    hipLaunchKernelGGL((tile_kernel<STAGE, CGW, S, false>), g, blk, 0, stream, a);
}

}  // namespace

hipError_t launch_a16_tile(int stage, const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  constexpr int S = MOE_TILE_STAGES;
  const int64_t grid = max_blocks * (a.N / 256);
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), blk(64 * (kComputeWaves + kLoaderWaves));
  if (stage == 1 && a.bm == 128) hipLaunchKernelGGL((a16_tile_kernel<1, 4, S>), g, blk, 0, stream, a);
  else if (stage == 1 && a.bm == 64) hipLaunchKernelGGL((a16_tile_kernel<1, 2, S>), g, blk, 0, stream, a);
  else if (stage == 1 && a.bm == 32) hipLaunchKernelGGL((a16_tile_kernel<1, 1, S>), g, blk, 0, stream, a);
  else if (stage == 2 && a.bm == 32) hipLaunchKernelGGL((a16_tile_kernel<2, 1, S>), g, blk, 0, stream, a);
  else if (stage == 2 && a.bm == 128) hipLaunchKernelGGL((a16_tile_kernel<2, 4, S>), g, blk, 0, stream, a);
  else if (stage == 2 && a.bm == 64) hipLaunchKernelGGL((a16_tile_kernel<2, 2, S>), g, blk, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tile(int stage, const GemmArgs& a, int64_t max_blocks, hipStream_t stream) {
  constexpr int S = MOE_TILE_STAGES;
  const int64_t grid = max_blocks * (a.N / 256);
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), blk(64 * (kComputeWaves + kLoaderWaves));
  if (stage == 1 && a.bm == 128) launch_one<1, 4, S>(a, g, blk, stream);
  else if (stage == 1 && a.bm == 64) launch_one<1, 2, S>(a, g, blk, stream);
  else if (stage == 2 && a.bm == 128) launch_one<2, 4, S>(a, g, blk, stream);
  else if (stage == 2 && a.bm == 64) launch_one<2, 2, S>(a, g, blk, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
