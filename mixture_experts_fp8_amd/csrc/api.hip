// C ABI of the A8W4 MoE library: argument checks, block size choice,
// workspace carving and the launch sequence.  Declarations and the contract
// of every entry point are in include/moe_a8w4.h.
#include <stdint.h>
#include <stddef.h>

#include <initializer_list>
#include <mutex>

#include "moe_a8w4.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

using moe::GemmArgs;

int check_dims(const moe_a8w4_dims* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->tokens < 0 || d->tokens >= (1 << 24)) return MOE_ERR_DIMS;
  if (d->hidden <= 0 || d->hidden % 512 != 0 || d->hidden > (1 << 20)) return MOE_ERR_DIMS;
  if (d->inter <= 0 || d->inter % 128 != 0 || d->inter > (1 << 20)) return MOE_ERR_DIMS;
  if (d->num_experts < 1 || d->num_experts > moe::kMaxExperts) return MOE_ERR_DIMS;
  if (d->topk < 1 || d->topk > moe::kMaxTopk) return MOE_ERR_DIMS;
  if (d->routed_experts < 0) return MOE_ERR_DIMS;
  return MOE_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Every pointer of a call 16-byte aligned, as the header requires (kernels
// read ids, codes and scales with 16-byte loads).
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : (int)e; }

bool valid_bm(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

// Mean routes per routed expert, the statistic the block size follows.  For
// a local slice of experts the router's routes spread over all the experts
// it chooses among (routed_experts > num_experts).  A layer that holds more
// experts than the router chooses among (routed_experts < num_experts) holds
// num_experts - routed_experts shared experts, each taking one of every
// token's top-k slots; those routes fill the shared experts' own blocks and
// are left out of the mean.
double routes_per_expert(const moe_a8w4_dims* d) {
  if (d->routed_experts > 0 && d->routed_experts < d->num_experts) {
    const int shared = d->num_experts - d->routed_experts;
    const int k = d->topk > shared ? d->topk - shared : d->topk;
    return (double)d->tokens * k / d->routed_experts;
  }
  const int experts = d->routed_experts > d->num_experts ? d->routed_experts : d->num_experts;
  return (double)d->tokens * d->topk / experts;
}

// Rows per sorted block from the mean number of routes per routed expert.
// Column groups of 16 past a block's last route are skipped by the GEMMs, so
// a larger block only costs padding; a smaller one re-reads an expert's
// weights once per extra block.
int choose_bm(const moe_a8w4_dims* d) {
  const double avg = routes_per_expert(d);
  if (avg <= 8.0) return 16;
  if (avg <= 20.0) return 32;   // local slice: 16 per expert, 32 beat 64 by 9 %; 24, 64 beat 32 by 8 %
  if (avg <= 40.0) return 64;
  return 128;
}

int64_t capacity(const moe_a8w4_dims* d, int bm) {
  const int64_t R = (int64_t)d->tokens * d->topk;
  const int64_t nexp = R < d->num_experts ? R : d->num_experts;
  const int64_t cap = R + nexp * (bm - 1);
  return (cap + bm - 1) / bm * bm;
}

// Route rows: [M, topk, H] 16-bit codes, then [M, topk, H/32] exponent bytes.
size_t route_codes_bytes(const moe_a8w4_dims* d) { return (size_t)d->tokens * d->topk * d->hidden * 2; }
size_t route_rows_bytes(const moe_a8w4_dims* d) {
  return route_codes_bytes(d) + (size_t)d->tokens * d->topk * (d->hidden / 32);
}

// int32 counters of the fused decode launch: status word (in a 256-byte run
// of its own), per-block stage-one counts (one 256-byte run each), per-block
// stage-two counts, per (token, stage-two column range) route counts (at
// most H/64 ranges).
int64_t fused_counters(const moe_a8w4_dims* d, int bm) {
  const int64_t blocks = capacity(d, bm) / bm;
  return moe::kCounterStride * (1 + blocks) + blocks + (int64_t)d->tokens * (d->hidden / 64);
}

bool fused_bm(int bm) { return bm == 16 || bm == 32; }

struct Layout {
  size_t aq, as, sorted, bexp, npad, iq, is, y, total;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(const moe_a8w4_dims* d, int bm) {
  const size_t M = d->tokens, H = d->hidden, I = d->inter;
  const size_t cap = (size_t)capacity(d, bm);
  Layout L;
  size_t o = 0;
  L.aq = o;     o += al256(M * H);
  L.as = o;     o += al256(M * H / 32);
  L.sorted = o; o += al256(cap * 4);
  L.bexp = o;   o += al256(cap / bm * 4);
  L.npad = o;   o += 256;
  L.iq = o;     o += al256(cap * I);
  L.is = o;     o += al256(cap * I / 32);
  L.y = o;      o += al256(route_rows_bytes(d));
  L.total = o;
  return L;
}

GemmArgs stage1_args(const moe_a8w4_dims* d, int bm, const uint8_t* a_q, const uint8_t* a_s,
                     const int32_t* sorted, const int32_t* bexp, const int32_t* npad,
                     const uint8_t* w, const uint8_t* ws, uint8_t* iq, uint8_t* is) {
  GemmArgs a = {};
  a.M = d->tokens; a.topk = d->topk; a.N = 2 * d->inter; a.K = d->hidden; a.bm = bm;
  a.sorted_ids = sorted; a.block_expert = bexp; a.num_padded = npad;
  a.bq = a_q; a.bs = a_s; a.w = w; a.ws = ws; a.out_q = iq; a.out_s = is;
  return a;
}

GemmArgs stage2_args(const moe_a8w4_dims* d, int bm, const uint8_t* iq, const uint8_t* is,
                     const int32_t* sorted, const int32_t* bexp, const int32_t* npad,
                     const float* wts, const uint8_t* w, const uint8_t* ws, void* y) {
  GemmArgs a = {};
  a.M = d->tokens; a.topk = d->topk; a.N = d->hidden; a.K = d->inter; a.bm = bm;
  a.sorted_ids = sorted; a.block_expert = bexp; a.num_padded = npad;
  a.bq = iq; a.bs = is; a.w = w; a.ws = ws; a.topk_weights = wts;
  a.y_codes = static_cast<int16_t*>(y);
  a.y_exps = static_cast<uint8_t*>(y) + route_codes_bytes(d);
  return a;
}

moe::FusedArgs fused_args(const moe_a8w4_dims* d, int bm, int32_t* cnt, const int32_t* topk_ids,
                          void* out) {
  moe::FusedArgs f = {};
  const int64_t blocks = capacity(d, bm) / bm;
  f.status = cnt;
  f.block_done = cnt + moe::kCounterStride;
  f.block_seen = cnt + moe::kCounterStride * (1 + blocks);
  f.token_done = f.block_seen + blocks;
  f.topk_ids = topk_ids;
  f.num_experts = d->num_experts;
  f.expert_offset = d->expert_offset;
  f.out = static_cast<uint16_t*>(out);
  return f;
}

// A16W4 variant: blocks of 16 routes while an expert averages at most 8 (the
// register-blocked kernel), then the LDS-tiled kernel in blocks of 32 up to
// 40, 64 up to 64 and 128 beyond.  Measured, 384 experts top-6: at 8 routes
// per expert the register kernel's blocks of 16 beat the tiled kernel's 32
// (447 against 487 us); at 32 blocks of 32 beat 64 (550 against 702); at 48
// blocks of 64 beat 32 (759 against 818); 16384 tokens: 2851 us in blocks of
// 64, 2515 in blocks of 128.
int a16_bm(const moe_a8w4_dims* d) {
  const double avg = routes_per_expert(d);
  return avg <= 8.0 ? 16 : avg <= 40.0 ? 32 : avg <= 64.0 ? 64 : 128;
}

struct A16Layout {
  size_t sorted, bexp, npad, inter, y, total;
};

// sort buffers, BF16 intermediate [capacity, I], route rows
A16Layout a16_layout(const moe_a8w4_dims* d, int bm) {
  const size_t cap = (size_t)capacity(d, bm);
  A16Layout L;
  size_t o = 0;
  L.sorted = o; o += al256(cap * 4);
  L.bexp = o;   o += al256(cap / bm * 4);
  L.npad = o;   o += 256;
  L.inter = o;  o += al256(cap * d->inter * 2);
  L.y = o;      o += al256(route_rows_bytes(d));
  L.total = o;
  return L;
}

GemmArgs a16_stage1_args(const moe_a8w4_dims* d, int bm, const void* hidden, const int32_t* sorted,
                         const int32_t* bexp, const int32_t* npad, const uint8_t* w, const uint8_t* ws,
                         void* inter) {
  GemmArgs a = {};
  a.M = d->tokens; a.topk = d->topk; a.N = 2 * d->inter; a.K = d->hidden; a.bm = bm;
  a.sorted_ids = sorted; a.block_expert = bexp; a.num_padded = npad;
  a.bq = static_cast<const uint8_t*>(hidden); a.w = w; a.ws = ws;
  a.out_q = static_cast<uint8_t*>(inter);
  return a;
}

}  // namespace

extern "C" {

int moe_a8w4_workspace_bytes(const moe_a8w4_dims* dims, size_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = layout(dims, choose_bm(dims)).total;
  return MOE_OK;
}

int moe_a8w4_block_m(const moe_a8w4_dims* dims) {
  int st = check_dims(dims);
  if (st) return st;
  return choose_bm(dims);
}

int64_t moe_a8w4_sort_capacity(const moe_a8w4_dims* dims, int32_t block_m) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_bm(block_m)) return MOE_ERR_BLOCK_M;
  return capacity(dims, block_m);
}

int moe_a8w4_pack_weights(const moe_a8w4_dims* dims, const uint8_t* w13, const uint8_t* w13_s,
                          const uint8_t* w2, const uint8_t* w2_s, uint8_t* w13_p, uint8_t* w13_s_p,
                          uint8_t* w2_p, uint8_t* w2_s_p, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  const void* ptrs[8] = {w13, w13_s, w2, w2_s, w13_p, w13_s_p, w2_p, w2_s_p};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned(p, 16)) return MOE_ERR_ALIGN;
  }
  const int64_t E = dims->num_experts, H = dims->hidden, I = dims->inter;
  hipError_t e = moe::launch_pack(w13, w13_s, w13_p, w13_s_p, E, 2 * I, H, stream);
  if (e != hipSuccess) return status_of(e);
  return status_of(moe::launch_pack(w2, w2_s, w2_p, w2_s_p, E, H, I, stream));
}

namespace {

// The layer after argument checks: prep (with the router when ra.logits is
// set; ids then comes from it), stage one, stage two, combine.
int forward_body(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                 const float* topk_weights, const moe::RouteArgs& ra, const uint8_t* w13_p,
                 const uint8_t* w13_s_p, const uint8_t* w2_p, const uint8_t* w2_s_p, void* out,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!aligned(workspace, 256)) return MOE_ERR_ALIGN;
  const int bm = choose_bm(dims);
  const Layout L = layout(dims, bm);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* a_q = ws + L.aq;
  uint8_t* a_s = ws + L.as;
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + L.bexp);
  int32_t* npad = reinterpret_cast<int32_t*>(ws + L.npad);
  uint8_t* iq = ws + L.iq;
  uint8_t* is = ws + L.is;
  uint8_t* y = ws + L.y;
  const int64_t max_blocks = capacity(dims, bm) / bm;

  // four launches: at every decode size they measured faster than prep +
  // moe_a8w4_stages_fused (the fused launch)
  hipError_t e = moe::launch_prep(topk_ids, dims->tokens, dims->topk, dims->num_experts,
                                  dims->expert_offset, bm, sorted, bexp, npad,
                                  static_cast<const uint16_t*>(hidden), dims->hidden, a_q, a_s, ra, stream);
  if (e != hipSuccess) return status_of(e);
  e = moe::launch_stage1(stage1_args(dims, bm, a_q, a_s, sorted, bexp, npad, w13_p, w13_s_p, iq, is),
                         max_blocks, stream);
  if (e != hipSuccess) return status_of(e);
  e = moe::launch_stage2(stage2_args(dims, bm, iq, is, sorted, bexp, npad, topk_weights, w2_p,
                                     w2_s_p, y), max_blocks, stream);
  if (e != hipSuccess) return status_of(e);
  return status_of(moe::launch_combine(dims->tokens, dims->hidden, dims->topk, dims->num_experts,
                                       dims->expert_offset, topk_ids, reinterpret_cast<int16_t*>(y),
                                       y + route_codes_bytes(dims), static_cast<uint16_t*>(out), stream));
}

// Router dims: 1 <= k_routed <= routed <= kMaxExperts, k_routed + shared
// slot <= kMaxTopk.
bool valid_route(int32_t routed, int32_t k_routed, int32_t shared_expert) {
  if (routed < 1 || routed > moe::kMaxExperts) return false;
  if (k_routed < 1 || k_routed > routed) return false;
  return k_routed + (shared_expert >= 0 ? 1 : 0) <= moe::kMaxTopk;
}

}  // namespace

int moe_a8w4_forward(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                     const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                     const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[9] = {hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p, out, workspace};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned(p, 16)) return MOE_ERR_ALIGN;
  }
  return forward_body(dims, hidden, topk_ids, topk_weights, moe::RouteArgs{}, w13_p, w13_s_p, w2_p,
                      w2_s_p, out, workspace, workspace_bytes, stream);
}

int moe_a8w4_route(int32_t M, int32_t routed_experts, int32_t k_routed, int32_t shared_expert,
                   const float* logits, int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (M < 0 || M >= (1 << 24) || !valid_route(routed_experts, k_routed, shared_expert)) return MOE_ERR_DIMS;
  if (M == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(topk_ids, 16) || !aligned(topk_weights, 16)) return MOE_ERR_ALIGN;
  const moe::RouteArgs ra{logits, routed_experts, k_routed, shared_expert, topk_ids, topk_weights};
  return status_of(moe::launch_route(ra, M, stream));
}

int moe_a8w4_forward_routed(const moe_a8w4_dims* dims, const void* hidden, const float* router_logits,
                            int32_t shared_expert, int32_t* topk_ids, float* topk_weights,
                            const uint8_t* w13_p, const uint8_t* w13_s_p, const uint8_t* w2_p,
                            const uint8_t* w2_s_p, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  const int32_t k_routed = dims->topk - (shared_expert >= 0 ? 1 : 0);
  if (!valid_route(dims->routed_experts, k_routed, shared_expert)) return MOE_ERR_DIMS;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[11] = {hidden, router_logits, topk_ids, topk_weights, w13_p, w13_s_p,
                          w2_p, w2_s_p, out, workspace, hidden};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned(p, 16)) return MOE_ERR_ALIGN;
  }
  const moe::RouteArgs ra{router_logits, dims->routed_experts, k_routed, shared_expert, topk_ids,
                          topk_weights};
  return forward_body(dims, hidden, topk_ids, topk_weights, ra, w13_p, w13_s_p, w2_p, w2_s_p, out,
                      workspace, workspace_bytes, stream);
}

int moe_a8w4_quant_act(int32_t M, int32_t H, const void* x, uint8_t* q, uint8_t* s,
                       hipStream_t stream) {
  if (M < 0 || H <= 0 || H % 32 != 0) return MOE_ERR_DIMS;
  if (M == 0) return MOE_OK;
  if (!x || !q || !s) return MOE_ERR_NULL;
  if (!all_aligned16({x, q, s})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_prep(nullptr, M, 1, 1, 0, 16, nullptr, nullptr, nullptr,
                                     static_cast<const uint16_t*>(x), H, q, s, moe::RouteArgs{}, stream));
}

int moe_a8w4_sort(const moe_a8w4_dims* dims, int32_t block_m, const int32_t* topk_ids,
                  int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                  hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_bm(block_m)) return MOE_ERR_BLOCK_M;
  if (!num_padded) return MOE_ERR_NULL;
  if (dims->tokens > 0 && (!topk_ids || !sorted_ids || !block_expert)) return MOE_ERR_NULL;
  if (!all_aligned16({topk_ids, sorted_ids, block_expert, num_padded})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_prep(topk_ids, dims->tokens, dims->topk, dims->num_experts,
                                    dims->expert_offset, block_m, sorted_ids, block_expert,
                                    num_padded, nullptr, 0, nullptr, nullptr, moe::RouteArgs{}, stream));
}

int moe_a8w4_quant_sort(const moe_a8w4_dims* dims, int32_t block_m, const void* hidden,
                        const int32_t* topk_ids, uint8_t* a_q, uint8_t* a_s, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_padded, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_bm(block_m)) return MOE_ERR_BLOCK_M;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[7] = {hidden, topk_ids, a_q, a_s, sorted_ids, block_expert, num_padded};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  if (!all_aligned16({hidden, topk_ids, a_q, a_s, sorted_ids, block_expert, num_padded})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_prep(topk_ids, dims->tokens, dims->topk, dims->num_experts,
                                    dims->expert_offset, block_m, sorted_ids, block_expert,
                                    num_padded, static_cast<const uint16_t*>(hidden), dims->hidden,
                                    a_q, a_s, moe::RouteArgs{}, stream));
}

int moe_a8w4_stage1(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* a_q,
                    const uint8_t* a_s, const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const uint8_t* w13_p, const uint8_t* w13_s_p,
                    uint8_t* inter_q, uint8_t* inter_s, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_bm(block_m)) return MOE_ERR_BLOCK_M;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[9] = {a_q, a_s, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_q, inter_s};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  if (!all_aligned16({a_q, a_s, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_q, inter_s}))
    return MOE_ERR_ALIGN;
  const int64_t max_blocks = capacity(dims, block_m) / block_m;
  return status_of(moe::launch_stage1(stage1_args(dims, block_m, a_q, a_s, sorted_ids, block_expert,
                                                  num_padded, w13_p, w13_s_p, inter_q, inter_s),
                                      max_blocks, stream));
}

int moe_a8w4_stage2(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* inter_q,
                    const uint8_t* inter_s, const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, const float* topk_weights, const uint8_t* w2_p,
                    const uint8_t* w2_s_p, void* y_routes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_bm(block_m)) return MOE_ERR_BLOCK_M;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[10] = {inter_q, inter_s, sorted_ids, block_expert, num_padded, topk_weights,
                          w2_p, w2_s_p, y_routes, inter_q};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  if (!all_aligned16({inter_q, inter_s, sorted_ids, block_expert, num_padded, topk_weights, w2_p, w2_s_p,
                      y_routes}))
    return MOE_ERR_ALIGN;
  const int64_t max_blocks = capacity(dims, block_m) / block_m;
  return status_of(moe::launch_stage2(stage2_args(dims, block_m, inter_q, inter_s, sorted_ids,
                                                  block_expert, num_padded, topk_weights, w2_p,
                                                  w2_s_p, y_routes),
                                      max_blocks, stream));
}

int moe_a8w4_combine(const moe_a8w4_dims* dims, const int32_t* topk_ids, const void* y_routes,
                     void* out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->tokens == 0) return MOE_OK;
  if (!topk_ids || !y_routes || !out) return MOE_ERR_NULL;
  if (!all_aligned16({topk_ids, y_routes, out})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_combine(dims->tokens, dims->hidden, dims->topk, dims->num_experts,
                                       dims->expert_offset, topk_ids,
                                       static_cast<const int16_t*>(y_routes),
                                       static_cast<const uint8_t*>(y_routes) + route_codes_bytes(dims),
                                       static_cast<uint16_t*>(out), stream));
}

int64_t moe_a8w4_fused_counters(const moe_a8w4_dims* dims, int32_t block_m) {
  int st = check_dims(dims);
  if (st) return st;
  if (!fused_bm(block_m)) return MOE_ERR_BLOCK_M;
  return fused_counters(dims, block_m);
}

int moe_a8w4_stages_fused(const moe_a8w4_dims* dims, int32_t block_m, const uint8_t* a_q,
                          const uint8_t* a_s, const int32_t* sorted_ids, const int32_t* block_expert,
                          const int32_t* num_padded, const int32_t* topk_ids, const float* topk_weights,
                          const uint8_t* w13_p, const uint8_t* w13_s_p, const uint8_t* w2_p,
                          const uint8_t* w2_s_p, uint8_t* inter_q, uint8_t* inter_s, void* y_routes,
                          int32_t* counters, void* out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!fused_bm(block_m)) return MOE_ERR_BLOCK_M;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[17] = {a_q, a_s, sorted_ids, block_expert, num_padded, topk_ids, topk_weights, w13_p,
                          w13_s_p, w2_p, w2_s_p, inter_q, inter_s, y_routes, counters, out, a_q};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  if (!all_aligned16({a_q, a_s, sorted_ids, block_expert, num_padded, topk_ids, topk_weights, w13_p, w13_s_p,
                      w2_p, w2_s_p, inter_q, inter_s, y_routes, counters, out}))
    return MOE_ERR_ALIGN;
  const int64_t max_blocks = capacity(dims, block_m) / block_m;
  return status_of(moe::launch_fused(
      stage1_args(dims, block_m, a_q, a_s, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_q,
                  inter_s),
      stage2_args(dims, block_m, inter_q, inter_s, sorted_ids, block_expert, num_padded, topk_weights,
                  w2_p, w2_s_p, y_routes),
      fused_args(dims, block_m, counters, topk_ids, out), max_blocks, stream));
}

// ------------------------------------------------------- A16W4 variant

int moe_a16w4_block_m(const moe_a8w4_dims* dims) {
  int st = check_dims(dims);
  if (st) return st;
  return a16_bm(dims);
}

int moe_a16w4_workspace_bytes(const moe_a8w4_dims* dims, size_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = a16_layout(dims, a16_bm(dims)).total;
  return MOE_OK;
}

int moe_a16w4_stage1(const moe_a8w4_dims* dims, int32_t block_m, const void* hidden,
                     const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                     const uint8_t* w13_p, const uint8_t* w13_s_p, void* inter_bf16, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_ERR_BLOCK_M;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[7] = {hidden, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_bf16};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  if (!all_aligned16({hidden, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_bf16}))
    return MOE_ERR_ALIGN;
  return status_of(moe::launch_a16_stage1(
      a16_stage1_args(dims, block_m, hidden, sorted_ids, block_expert, num_padded, w13_p, w13_s_p, inter_bf16),
      capacity(dims, block_m) / block_m, stream));
}

int moe_a16w4_forward(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                      const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                      const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[9] = {hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p, out, workspace};
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL;
  const void* al[7] = {hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, out};
  for (const void* p : al)
    if (!aligned(p, 16)) return MOE_ERR_ALIGN;
  if (!aligned(w2_s_p, 16) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  const int bm = a16_bm(dims);
  const A16Layout L = a16_layout(dims, bm);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + L.bexp);
  int32_t* npad = reinterpret_cast<int32_t*>(ws + L.npad);
  uint8_t* inter = ws + L.inter;
  uint8_t* y = ws + L.y;
  const int64_t max_blocks = capacity(dims, bm) / bm;
  // the sort alone (no activation quantiser), stage one, stage two, combine
  hipError_t e = moe::launch_prep(topk_ids, dims->tokens, dims->topk, dims->num_experts,
                                  dims->expert_offset, bm, sorted, bexp, npad, nullptr, 0, nullptr,
                                  nullptr, moe::RouteArgs{}, stream);
  if (e != hipSuccess) return status_of(e);
  e = moe::launch_a16_stage1(
      a16_stage1_args(dims, bm, hidden, sorted, bexp, npad, w13_p, w13_s_p, inter), max_blocks, stream);
  if (e != hipSuccess) return status_of(e);
  GemmArgs a2 = stage2_args(dims, bm, inter, nullptr, sorted, bexp, npad, topk_weights, w2_p, w2_s_p, y);
  e = moe::launch_a16_stage2(a2, max_blocks, stream);
  if (e != hipSuccess) return status_of(e);
  return status_of(moe::launch_combine(dims->tokens, dims->hidden, dims->topk, dims->num_experts,
                                       dims->expert_offset, topk_ids, reinterpret_cast<int16_t*>(y),
                                       y + route_codes_bytes(dims), static_cast<uint16_t*>(out), stream));
}

int moe_a8w4_mfma_probe(int64_t n, int32_t byte_sel, const uint8_t* a_fp4, const uint8_t* a_scale,
                        const uint8_t* b_fp8, const uint8_t* b_scale, float* d, hipStream_t stream) {
  if (n < 0 || n > (1 << 24) || byte_sel < 0 || byte_sel > 3) return MOE_ERR_DIMS;
  if (n == 0) return MOE_OK;
  if (!a_fp4 || !a_scale || !b_fp8 || !b_scale || !d) return MOE_ERR_NULL;
  if (!aligned(a_fp4, 16) || !aligned(b_fp8, 16) || !aligned(d, 4)) return MOE_ERR_ALIGN;
  return status_of(moe::launch_mfma_probe(n, byte_sel, a_fp4, a_scale, b_fp8, b_scale, d, stream));
}

int moe_a8w4_stream_probe(int32_t layout, int64_t rows, int32_t K, const uint8_t* w, const uint8_t* w_s,
                          uint32_t* out, hipStream_t stream) {
  if ((layout != 0 && layout != 1) || rows < 0 || rows % 64 || rows > ((int64_t)1 << 28) || K <= 0 ||
      K % 512 || K > (1 << 16))
    return MOE_ERR_DIMS;
  if (rows == 0) return MOE_OK;
  if (!w || !w_s || !out) return MOE_ERR_NULL;
  if (!all_aligned16({w, w_s, out})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_stream_probe(layout, rows / 64, K, w, w_s, out, stream));
}

int moe_a16w4_mfma_probe(int64_t n, const void* a_bf16, const void* b_bf16, float* d, hipStream_t stream) {
  if (n < 0 || n > (1 << 24)) return MOE_ERR_DIMS;
  if (n == 0) return MOE_OK;
  if (!a_bf16 || !b_bf16 || !d) return MOE_ERR_NULL;
  if (!all_aligned16({a_bf16, b_bf16, d})) return MOE_ERR_ALIGN;
  return status_of(moe::launch_mfma_bf16_probe(n, static_cast<const uint16_t*>(a_bf16),
                                               static_cast<const uint16_t*>(b_bf16), d, stream));
}

}  // extern "C"

// ------------------------------------------------- the no-allocation form
//
// moe_a8w4_forward_noalloc takes its workspace from this array instead of a
// caller buffer.  In host code `scratch` names a host-side stand-in, not the
// device copy: its device address is looked up once per device (with that
// device current) and only that address is passed to kernels.
namespace {

static __device__ __align__(256) uint8_t scratch[MOE_A8W4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
int current_scratch(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return status_of(e);
  if (dev < 0 || dev >= kMaxDevices) return status_of(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return status_of(e);
    if (!ptr) return status_of(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_a8w4_forward_noalloc(const moe_a8w4_dims* dims, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const uint8_t* w13_p, const uint8_t* w13_s_p,
                             const uint8_t* w2_p, const uint8_t* w2_s_p, void* out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->tokens == 0) return MOE_OK;
  const void* ptrs[8] = {hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p, out};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned(p, 16)) return MOE_ERR_ALIGN;
  }
  // nothing of the workspace has to start at zero: every byte a call reads
  // was written earlier in the same call
  if (layout(dims, choose_bm(dims)).total > MOE_A8W4_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st) return st;
  return forward_body(dims, hidden, topk_ids, topk_weights, moe::RouteArgs{}, w13_p, w13_s_p, w2_p, w2_s_p, out,
                      ws, MOE_A8W4_NOALLOC_SCRATCH_BYTES, stream);
}

const char* moe_a8w4_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_DIMS: return "a dimension is outside the supported limits";
    case MOE_ERR_ALIGN: return "a pointer is misaligned (16 B; workspace 256 B)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_a8w4_workspace_bytes()";
    case MOE_ERR_BLOCK_M: return "block_m must be 16, 32, 64 or 128";
    case MOE_ERR_SCRATCH: return "the call needs more than MOE_A8W4_NOALLOC_SCRATCH_BYTES of scratch";
    default: return status > 0 ? "HIP launch error (value is a hipError_t)" : "unknown status";
  }
}

}  // extern "C"
