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
// One workgroup of 16 waves.  Wave w owns the contiguous routes
// [w C, (w+1) C), C = ceil(R / 16):
//   1. each wave counts its routes per expert (LDS atomics; counts only);
//   2. one scan gives every expert its padded start and every (wave, expert)
//      the offset of that wave's first route of the expert;
//   3. each wave walks its chunk 64 routes at a time; the rank of a route
//      among same-expert routes of the piece is a popcount of a wave-private
//      64-bit lane mask (ds_or_b64), so no barrier or atomic ordering is
//      involved and the result is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kSortWaves = kPrepThreads / kWave;

struct SortSmem {
  int cnt[kSortWaves][kMaxExperts];                 // per-wave counts, then running offsets
  unsigned long long mask[kSortWaves][kMaxExperts]; // per-wave lane masks of one 64-route piece
  int wave_total[kSortWaves];
};

// Orders this wave's LDS accesses before and after (all lanes of a wave run
// in lockstep; the fences keep the compiler from reordering across this point
// and make it wait for the outstanding LDS operations).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ void sort_block(SortSmem& sm, const int32_t* __restrict__ ids, int M, int topk, int E,
                           int expert_offset, int bm, int32_t* __restrict__ sorted_ids,
                           int32_t* __restrict__ block_expert, int32_t* __restrict__ num_padded) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = M * topk;
  const int C = (R + kSortWaves - 1) / kSortWaves;
  const int f0 = w * C, f1 = min(R, f0 + C);

  for (int i = tid; i < kSortWaves * kMaxExperts; i += kPrepThreads) {
    (&sm.cnt[0][0])[i] = 0;
    (&sm.mask[0][0])[i] = 0ull;
  }
  __syncthreads();

  // 1. per-wave histogram of local routes
  for (int f = f0 + lane; f < f1; f += 64) {
    const int le = ids[f] - expert_offset;
    if ((unsigned)le < (unsigned)E) atomicAdd(&sm.cnt[w][le], 1);
  }
  __syncthreads();

  // 2. one expert per thread: its count, padded size, and the waves' offsets
  int c = 0;
  if (tid < E) {
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
    int run = start;
    for (int j = 0; j < kSortWaves; ++j) {  // counts become each wave's first position
      const int n = sm.cnt[j][tid];
      sm.cnt[j][tid] = run;
      run += n;
    }
    for (int p = start + c; p < start + pc; ++p) sorted_ids[p] = M;
    for (int b = start / bm; b < (start + pc) / bm; ++b) block_expert[b] = tid;
  }
  if (tid == 0) *num_padded = total;
  __syncthreads();

  // 3. each wave places its own routes in order; only wave-private LDS is used
  const unsigned long long bit = 1ull << lane;
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    int le = -1;
    if (f < f1) {
      le = ids[f] - expert_offset;
      if ((unsigned)le >= (unsigned)E) le = -1;
    }
    if (le >= 0) atomicOr(&sm.mask[w][le], bit);
    wave_sync();
    unsigned long long m = 0;
    int rank = 0;
    if (le >= 0) {
      m = sm.mask[w][le];
      rank = __popcll(m & (bit - 1));
      const int t = f / topk, k = f - t * topk;
      sorted_ids[sm.cnt[w][le] + rank] = (k << kSentinelShift) | t;
    }
    wave_sync();
    if (le >= 0 && rank == 0) {
      sm.cnt[w][le] += __popcll(m);
      sm.mask[w][le] = 0ull;
    }
    wave_sync();
  }
}

// Four lanes own one 32-element block: lane i of the quad loads 8 BF16 values
// (16 B), so a wave reads 1 KB contiguous per load and writes 512 B of codes.
// FP8 activations with one E8M0 scale per 1x32 block (aiter PR 5609,
// Configuration).  n8 and the stride are multiples of 4, so a quad is either
// all in range or all out.
__device__ void quant_range(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                            uint8_t* __restrict__ s, int64_t n8, int64_t first, int64_t stride) {
  for (int64_t i = first; i < n8; i += stride) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + i * 8);
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
}

// Workgroup 0 sorts (if ids != nullptr); workgroups 1.. quantise (if x != nullptr).
__global__ void __launch_bounds__(kPrepThreads) prep_kernel(
    const int32_t* __restrict__ ids, int M, int topk, int E, int expert_offset, int bm,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded, const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, int64_t n8) {
  __shared__ SortSmem sm;
  if (blockIdx.x == 0) {
    if (ids) sort_block(sm, ids, M, topk, E, expert_offset, bm, sorted_ids, block_expert, num_padded);
    return;
  }
  quant_range(x, q, s, n8, (int64_t)(blockIdx.x - 1) * kPrepThreads + threadIdx.x,
              (int64_t)(gridDim.x - 1) * kPrepThreads);
}

int quant_blocks(int64_t n8) {
  int64_t b = (n8 + kPrepThreads - 1) / kPrepThreads;
  return (int)(b > 1024 ? 1024 : b);
}

}  // namespace

hipError_t launch_prep(const int32_t* ids, int32_t M, int32_t topk, int32_t E, int32_t expert_offset,
                       int32_t bm, int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                       const uint16_t* x, int64_t H, uint8_t* q, uint8_t* s, hipStream_t stream) {
  const int64_t n8 = x ? (int64_t)M * H / 8 : 0;
  const int grid = 1 + (n8 > 0 ? quant_blocks(n8) : 0);
  if (!ids && grid == 1) return hipSuccess;
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(kPrepThreads), 0, stream, ids, M, topk, E,
                     expert_offset, bm, sorted_ids, block_expert, num_padded, x, q, s, n8);
  return hipGetLastError();
}

}  // namespace moe
