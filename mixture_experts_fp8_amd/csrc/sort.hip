// Route sort of the A8W4 MoE layer: groups the top-k routes by local expert
// into blocks of block_m rows, padded with a sentinel, with one expert id per
// block.  Sorting is part of the timed fused-MoE call (aiter PR 5904, "Add
// tuned a8w4 fused-MoE configs for DeepSeek V4.1-Flash (TP4 + EP, gfx950)",
// "Fused-MoE kernel, expert-parallel benchmark"); the sort block must equal
// the stage-two tile (aiter PR 5609, "Add DeepSeek V4.1 Flash TP4 gfx950 MoE
// tuning", the CSV layout test under "Commands run").
//
// Output order (a fixed convention shared with the test oracle): experts in
// ascending local id, an expert's routes in ascending flat index t*topk + k,
// each route written as (k << 24) | t, each expert's run padded with the
// value M up to a multiple of block_m; experts with no route get no block.
// Routes whose expert lies outside [expert_offset, expert_offset + E) are
// dropped.
//
// One workgroup of 1024 threads: LDS histogram, a workgroup scan of the
// padded counts, then placement in rounds of 1024 routes.  Within a round the
// rank of a route among same-expert routes comes from per-wave 64-bit lane
// masks (ds_or_b64) and popcounts, so the result is deterministic without any
// ordering of atomics.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;

__global__ void __launch_bounds__(kSortThreads) sort_kernel(const int32_t* __restrict__ ids, int M,
                                                            int topk, int E, int expert_offset,
                                                            int bm, int32_t* __restrict__ sorted_ids,
                                                            int32_t* __restrict__ block_expert,
                                                            int32_t* __restrict__ num_padded) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int cursor[kMaxExperts];
  __shared__ unsigned long long masks[kSortWaves][kMaxExperts];
  __shared__ int wave_total[kSortWaves];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = M * topk;

  for (int e = tid; e < kMaxExperts; e += kSortThreads) cnt[e] = 0;
  for (int i = tid; i < kSortWaves * kMaxExperts; i += kSortThreads) (&masks[0][0])[i] = 0ull;
  __syncthreads();

  // histogram of local routes
  for (int f = tid; f < R; f += kSortThreads) {
    const int le = ids[f] - expert_offset;
    if ((unsigned)le < (unsigned)E) atomicAdd(&cnt[le], 1);
  }
  __syncthreads();

  // exclusive scan of the block-padded counts (one expert per thread, E <= 512)
  const int c = (tid < E) ? cnt[tid] : 0;
  const int pc = (c + bm - 1) / bm * bm;
  int v = pc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wave_total[w] = v;
  __syncthreads();
  int before = 0, total = 0;
  for (int j = 0; j < kSortWaves; ++j) {
    const int t = wave_total[j];
    before += (j < w) ? t : 0;
    total += t;
  }
  const int start = before + v - pc;
  if (tid < E) {
    cursor[tid] = start;
    for (int p = start + c; p < start + pc; ++p) sorted_ids[p] = M;
    for (int b = start / bm; b < (start + pc) / bm; ++b) block_expert[b] = tid;
  }
  if (tid == 0) *num_padded = total;
  __syncthreads();

  // stable placement, 1024 routes per round
  const unsigned long long bit = 1ull << lane;
  for (int base = 0; base < R; base += kSortThreads) {
    const int f = base + tid;
    int le = -1;
    if (f < R) {
      le = ids[f] - expert_offset;
      if ((unsigned)le >= (unsigned)E) le = -1;
    }
    if (le >= 0) atomicOr(&masks[w][le], bit);
    __syncthreads();
    unsigned long long m = 0;
    int rank = 0;
    if (le >= 0) {
      m = masks[w][le];
      rank = __popcll(m & (bit - 1));
      int prior = 0;
      for (int j = 0; j < w; ++j) prior += __popcll(masks[j][le]);
      const int t = f / topk, k = f - t * topk;
      sorted_ids[cursor[le] + prior + rank] = (k << kSentinelShift) | t;
    }
    __syncthreads();
    if (le >= 0 && rank == 0) {
      atomicAdd(&cursor[le], __popcll(m));
      masks[w][le] = 0ull;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_sort(const int32_t* ids, int32_t M, int32_t topk, int32_t E, int32_t expert_offset,
                       int32_t bm, int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                       hipStream_t stream) {
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSortThreads), 0, stream, ids, M, topk, E,
                     expert_offset, bm, sorted_ids, block_expert, num_padded);
  return hipGetLastError();
}

}  // namespace moe
