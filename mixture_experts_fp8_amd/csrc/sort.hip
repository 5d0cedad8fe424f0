// Route sort of the A8W4 MoE layer, and the launch that runs it beside the
// per-1x32 FP8 activation quantiser.
//
// The sort groups the top-k routes by local expert into blocks of block_m
// rows, padded with a sentinel, with one expert id per block.  Sorting is part
// of the timed fused-MoE call (aiter PR 5904, "Add tuned a8w4 fused-MoE
// configs for DeepSeek V4.1-Flash (TP4 + EP, gfx950)", "Fused-MoE kernel,
// expert-parallel benchmark"); the sort block must equal the stage-two tile
// (aiter PR 5609, "Add DeepSeek V4.1 Flash TP4 gfx950 MoE tuning", the CSV
// layout test under "Commands run").
//
// Output order (a fixed convention shared with the test oracle): experts in
// ascending local id, an expert's routes in ascending flat index t*topk + k,
// each route written as (k << 24) | t, each expert's run padded with the
// value M up to a multiple of block_m; experts with no route get no block.
// Routes whose expert lies outside [expert_offset, expert_offset + E) are
// dropped.
//
// The routes are cut into NS contiguous chunks, one workgroup of 16 waves
// per chunk (NS = 1 up to 1024 routes, at most 64).  Every workgroup counts all routes per
// expert (so each knows every expert's padded start and how many of the
// expert's routes lie in earlier chunks; no data passes between workgroups),
// then places its own chunk.  Wave w of a workgroup owns the contiguous
// routes [w C, (w+1) C) of the chunk, C = ceil(chunk / 16):
//   1. count: per expert in total, before this chunk, and per wave of it
//      (LDS atomics; counts only);
//   2. one scan gives every expert its padded start and every (wave, expert)
//      the position of that wave's first route of the expert;
//   3. the padding and block experts.  At blocks of 16 (at most 15 padding
//      entries per expert) one lane per expert writes them.  At larger
//      blocks one wave per expert does, its lanes on consecutive positions,
//      the experts spread over every workgroup's waves: one lane per expert
//      writing up to block_m - 1 entries one at a time makes every store
//      touch 64 scattered lines (the sort of 28,672 routes in blocks of 128
//      took 25 us that way, 12 us with the per-wave stores).  At blocks of
//      16 the per-wave loop (up to 24 experts per wave in one workgroup) is
//      the slower one;
//   4. each wave walks its routes 64 at a time; the lanes holding the same
//      expert are found with one ballot per bit of the expert id, and the
//      rank of a route among them is a popcount of that lane mask, so no
//      barrier or atomic ordering is involved and the result is
//      deterministic.
// Workgroup 0 also writes num_padded.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kSortWaves = kPrepThreads / kWave;

constexpr int kRoutesPerSortBlock = 1024;
constexpr int kMaxSortBlocks = 64;

struct SortSmem {
  int cnt[kSortWaves][kMaxExperts];                 // per-wave counts, then running offsets
  int before[kMaxExperts];                          // routes per expert in earlier chunks
  int after[kMaxExperts];                           // and in later chunks
  int wave_total[kSortWaves];
};

int sort_blocks(int64_t R) {
  const int64_t n = (R + kRoutesPerSortBlock - 1) / kRoutesPerSortBlock;
  return (int)(n < 1 ? 1 : (n > kMaxSortBlocks ? kMaxSortBlocks : n));
}

// Orders this wave's LDS accesses before and after (all lanes of a wave run
// in lockstep; the fences keep the compiler from reordering across this point
// and make it wait for the outstanding LDS operations).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ void sort_chunk(SortSmem& sm, const int32_t* ids, int M, int topk, int E,
                           int expert_offset, int bm, int chunk, int nchunks,
                           int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                           int32_t* __restrict__ num_padded) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = M * topk;
  const int CH = (R + nchunks - 1) / nchunks;
  const int g0 = min(R, chunk * CH), g1 = min(R, g0 + CH);
  const int C = (g1 - g0 + kSortWaves - 1) / kSortWaves;
  const int f0 = g0 + w * C, f1 = min(g1, f0 + C);

  for (int i = tid; i < kSortWaves * kMaxExperts; i += kPrepThreads) (&sm.cnt[0][0])[i] = 0;
  for (int i = tid; i < kMaxExperts; i += kPrepThreads) {
    sm.before[i] = 0;
    sm.after[i] = 0;
  }
  __syncthreads();

  // 1. counts over all routes: before this chunk, per owning wave, after it
  // (one LDS atomic per route).  Each thread reads 16 B of ids per load and
  // has the next U loads in flight while it counts the current ones.
  auto count = [&](int f, int le) {
    if ((unsigned)le < (unsigned)E) {
      if (f < g0) atomicAdd(&sm.before[le], 1);
      else if (f < g1) atomicAdd(&sm.cnt[(f - g0) / C][le], 1);
      else atomicAdd(&sm.after[le], 1);
    }
  };
  constexpr int U = 4;
  const int R4 = R / 4;   // whole 16-byte groups of ids
  const int4* ids4 = reinterpret_cast<const int4*>(ids);
  auto load4 = [&](int4 (&v)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * kPrepThreads + tid;
      v[u] = j < R4 ? ids4[j] : make_int4(-1, -1, -1, -1);
    }
  };
  int4 nxt[U];
  load4(nxt, 0);
  for (int base = 0; base < R4; base += U * kPrepThreads) {
    int4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = nxt[u];
    if (base + U * kPrepThreads < R4) load4(nxt, base + U * kPrepThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * kPrepThreads + tid;
      if (j < R4) {
        count(4 * j, v[u].x - expert_offset);
        count(4 * j + 1, v[u].y - expert_offset);
        count(4 * j + 2, v[u].z - expert_offset);
        count(4 * j + 3, v[u].w - expert_offset);
      }
    }
  }
  if (tid < R - 4 * R4) count(4 * R4 + tid, ids[4 * R4 + tid] - expert_offset);
  __syncthreads();

  // 2. one expert per thread: its count, padded size, and the waves' offsets
  int c = 0;
  if (tid < E) {
    c = sm.before[tid] + sm.after[tid];
    for (int j = 0; j < kSortWaves; ++j) c += sm.cnt[j][tid];
  }
  const int pc = (c + bm - 1) / bm * bm;
  int v = pc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) sm.wave_total[w] = v;
  __syncthreads();
  int before = 0, total = 0;
  for (int j = 0; j < kSortWaves; ++j) {
    const int t = sm.wave_total[j];
    before += (j < w) ? t : 0;
    total += t;
  }
  const int start = before + v - pc;
  if (tid < E) {
    int run = start + sm.before[tid];
    for (int j = 0; j < kSortWaves; ++j) {  // counts become each wave's first position
      const int n = sm.cnt[j][tid];
      sm.cnt[j][tid] = run;
      run += n;
    }
    if (bm <= 16) {
      // blocks of 16: at most 15 padding entries, one lane per expert
      if (chunk == 0) {
        for (int p = start + c; p < start + pc; ++p) sorted_ids[p] = M;
        for (int b = start / bm; b < (start + pc) / bm; ++b) block_expert[b] = tid;
      }
    } else {
      // only this thread reads these two entries: they now hold the
      // expert's padded start and its route count
      sm.before[tid] = start;
      sm.after[tid] = c;
    }
  }
  if (chunk == 0 && tid == 0) *num_padded = total;
  __syncthreads();

  // 3. (blocks of 32 and more) the padding and the block experts: one wave
  // per expert, its lanes on consecutive positions (whole-line stores), the
  // experts spread over the waves of every sort workgroup
  if (bm > 16) {
    for (int e = chunk * kSortWaves + w; e < E; e += nchunks * kSortWaves) {
      const int st = sm.before[e], ce = sm.after[e];
      const int end = st + (ce + bm - 1) / bm * bm;
      for (int p = st + ce + lane; p < end; p += kWave) sorted_ids[p] = M;
      for (int b = st / bm + lane; b < end / bm; b += kWave) block_expert[b] = e;
    }
  }

  // 4. each wave places its own routes in order; only wave-private LDS is used
  static_assert(kMaxExperts <= 1023, "expert key needs more bits");
  const unsigned long long below = (1ull << lane) - 1;
  auto local_id = [&](int f) {
    int le = -1;
    if (f < f1) {
      le = ids[f] - expert_offset;
      if ((unsigned)le >= (unsigned)E) le = -1;
    }
    return le;
  };
  int le_next = local_id(f0 + lane);   // one piece of 64 ahead
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    const int le = le_next;
    le_next = local_id(base + 64 + lane);
    const int key = le + 1;   // 0 for no local route
    unsigned long long same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool on = (key >> bit) & 1;
      const unsigned long long m = __ballot(on);
      same &= on ? m : ~m;
    }
    const int rank = __popcll(same & below);
    if (le >= 0) {
      const int t = f / topk, k = f - t * topk;
      sorted_ids[sm.cnt[w][le] + rank] = (k << kSentinelShift) | t;
    }
    wave_sync();
    if (le >= 0 && rank == 0) sm.cnt[w][le] += __popcll(same);
    wave_sync();
  }
}

// Four lanes own one 32-element block: lane i of the quad loads 8 BF16 values
// (16 B), so a wave reads 1 KB contiguous per load and writes 512 B of codes.
// FP8 activations with one E8M0 scale per 1x32 block (aiter PR 5609,
// Configuration).  Each thread has U loads in flight.  n8 and the stride are
// multiples of 4, so a quad is either all in range or all out.
__device__ __forceinline__ void quant_one(uint4 raw, int64_t i, uint8_t* __restrict__ q,
                                          uint8_t* __restrict__ s) {
  float v[8];
  v[0] = bf16_to_f32(raw.x & 0xFFFFu); v[1] = bf16_to_f32(raw.x >> 16);
  v[2] = bf16_to_f32(raw.y & 0xFFFFu); v[3] = bf16_to_f32(raw.y >> 16);
  v[4] = bf16_to_f32(raw.z & 0xFFFFu); v[5] = bf16_to_f32(raw.z >> 16);
  v[6] = bf16_to_f32(raw.w & 0xFFFFu); v[7] = bf16_to_f32(raw.w >> 16);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int E = block_exponent(amax);
  *reinterpret_cast<uint2*>(q + i * 8) = encode8(v, exp2_neg(E));
  if ((i & 3) == 0) s[i >> 2] = (uint8_t)(E + 127);
}

__device__ void quant_range(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                            uint8_t* __restrict__ s, int64_t n8, int64_t first, int64_t stride) {
  constexpr int U = 4;
  int64_t i = first;
  for (; i + (U - 1) * stride < n8; i += U * stride) {
    v4i raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(x + (i + u * stride) * 8));
#pragma unroll
    for (int u = 0; u < U; ++u)
      quant_one(make_uint4(raw[u].x, raw[u].y, raw[u].z, raw[u].w), i + u * stride, q, s);
  }
  for (; i < n8; i += stride) quant_one(*reinterpret_cast<const uint4*>(x + i * 8), i, q, s);
}

// Router (backbone configurations: softmax top-k of the router logits,
// renormalised; the prefill configuration's fused shared expert in a last
// slot with weight 1).  One wave per token: lane l holds logits l, l + 64,
// ...; k rounds of a wave-wide arg-max (equal values: the lower expert id),
// then the weights as the softmax of the chosen logits -- the full softmax
// renormalised over the chosen ones, which is the same in exact arithmetic.
constexpr int kRouterPerLane = kMaxExperts / kWave;
// tokens the sort workgroup routes itself (one per wave) before sorting; for
// more, a launch of its own (a wave per token) costs less than the waves of
// one workgroup routing several tokens each
constexpr int kRouteInSortTokens = kSortWaves;

__device__ void route_token(const RouteArgs& ra, int64_t t) {
  const int lane = threadIdx.x & 63;
  const int Er = ra.routed, kr = ra.k_routed;
  const int k = kr + (ra.shared >= 0 ? 1 : 0);
  const float* l = ra.logits + t * Er;
  float v[kRouterPerLane];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < kRouterPerLane; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < Er ? l[e] : 0.f;
    if (e < Er) avail |= 1u << i;
  }
  constexpr int kNone = 0x7FFFFFFF;
  float my_v = 0.f, top0 = 0.f, ex = 0.f, sum = 0.f;
  int my_id = 0;
  for (int s = 0; s < kr; ++s) {
    float bv = 0.f;
    int bi = kNone;
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i)   // ascending id: > keeps the lower one
      if (((avail >> i) & 1u) && (bi == kNone || v[i] > bv)) {
        bv = v[i];
        bi = lane + kWave * i;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != kNone && (bi == kNone || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) avail &= ~(1u << (bi / kWave));
    if (s == 0) top0 = bv;
    const float es = expf(bv - top0);   // every lane: the sum runs in slot order
    sum += es;
    if (lane == s) {
      my_v = es;
      my_id = bi;
    }
  }
  ex = my_v;
  if (lane < kr) {
    ra.ids[t * k + lane] = my_id;
    ra.weights[t * k + lane] = ex / sum;
  } else if (lane == kr && ra.shared >= 0) {
    ra.ids[t * k + kr] = ra.shared;
    ra.weights[t * k + kr] = 1.0f;
  }
}

__global__ void __launch_bounds__(256) route_kernel(RouteArgs ra, int M) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < M) route_token(ra, t);
}

// Quantiser workgroups: one thread per 8 elements, at most 1024 workgroups
// (each thread then loops), or 4096 above 4M threads' worth, where the wider
// grid measured faster (prefill-shared 16384 tokens: 45 -> 39 us; at 4096
// tokens the 1024 cap is 1 us faster).
int quant_blocks(int64_t n8) {
  const int64_t b = (n8 + kPrepThreads - 1) / kPrepThreads;
  const int64_t cap = n8 > (int64_t(4) << 20) ? 4096 : 1024;
  return (int)(b > cap ? cap : b);
}

// Workgroups 0 .. ns-1 sort (ns = 0 without ids); the others quantise.  With
// ra.logits set (and ns = 1) the sort workgroup first routes every token,
// writing the ids it then sorts.
__global__ void __launch_bounds__(kPrepThreads) prep_kernel(
    const int32_t* ids, int M, int topk, int E, int expert_offset, int bm, int ns,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded, const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, int64_t n8, RouteArgs ra) {
  __shared__ SortSmem sm;
  if ((int)blockIdx.x < ns) {
    if (ra.logits) {
      for (int t = threadIdx.x >> 6; t < M; t += kSortWaves) route_token(ra, t);
      // the ids are read back by this workgroup only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    sort_chunk(sm, ids, M, topk, E, expert_offset, bm, blockIdx.x, ns, sorted_ids, block_expert,
               num_padded);
    return;
  }
  quant_range(x, q, s, n8, (int64_t)(blockIdx.x - ns) * kPrepThreads + threadIdx.x,
              (int64_t)(gridDim.x - ns) * kPrepThreads);
}

}  // namespace

hipError_t launch_route(const RouteArgs& ra, int32_t M, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, ra, M);
  return hipGetLastError();
}

hipError_t launch_prep(const int32_t* ids, int32_t M, int32_t topk, int32_t E, int32_t expert_offset,
                       int32_t bm, int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                       const uint16_t* x, int64_t H, uint8_t* q, uint8_t* s, const RouteArgs& ra,
                       hipStream_t stream) {
  const int64_t n8 = x ? (int64_t)M * H / 8 : 0;
  RouteArgs fused = ra;
  if (ra.logits) {
    ids = ra.ids;
    if (sort_blocks((int64_t)M * topk) > 1 || M > kRouteInSortTokens) {
      // several sort workgroups each read every id, or more tokens than the
      // sort workgroup's waves route quickly: route first
      hipError_t e = launch_route(ra, M, stream);
      if (e != hipSuccess) return e;
      fused.logits = nullptr;
    }
  }
  const int ns = ids ? sort_blocks((int64_t)M * topk) : 0;
  const int grid = ns + (n8 > 0 ? quant_blocks(n8) : 0);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(kPrepThreads), 0, stream, ids, M, topk, E,
                     expert_offset, bm, ns, sorted_ids, block_expert, num_padded, x, q, s, n8, fused);
  return hipGetLastError();
}

}  // namespace moe
