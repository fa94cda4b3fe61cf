// Host-side launchers of the MoE decode-layer kernels (internal interface
// between the C ABI in abi.hip and the kernel files).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Device arrays written by the route-compaction stage: the N*k (token, slot)
// routes grouped by expert, experts in ascending id, routes of one expert in
// ascending (token, slot).
struct Compact {
  int32_t *n_active;  // [1] number of experts with at least one route
  int32_t *active;    // [min(E, N*k)] expert id of each active slot
  int32_t *off;       // [min(E, N*k) + 1] first route position of each slot
  int32_t *route_tok; // [N*k] token of the route at a position
  int32_t *route_src; // [N*k] t*k + j of the route at a position
  int32_t *route_pos; // [N*k] position of route t*k + j (-1: dropped)
};

// logits[N, E] = x[N, h] . W[E, h]^T   (act_f32: fp32 operands, else bf16)
hipError_t launch_router(bool act_f32, const void *x, const void *W, float *logits, int N, int E,
                         int h, hipStream_t s);

// Top-k of every logits row (do_topk) and / or route compaction of idx (do_compact).
hipError_t launch_route(const float *logits, const float *bias, int32_t *idx, float *w, int N,
                        int E, int k, int scoring, int norm, float rsf, bool do_topk,
                        bool do_compact, const Compact &c, hipStream_t s);

// One streaming GEMV pass over the active experts (and the shared expert).
struct GemvArgs {
  const void *const *w0;  // routed weight tables [E]: gate (gate+up pass) or down
  const void *const *w1;  // up (gate+up pass) or NULL
  const void *const *s0;  // scale tables or NULL
  const void *const *s1;
  const void *sh_w0, *sh_w1, *sh_s0, *sh_s1;  // shared expert (sh_w0 NULL = none)
  int rows, K;        // routed matrix: rows x K
  int sh_rows, sh_K;  // shared matrix
  const void *src;    // gate+up: x [N, h] (act dtype); down: act [N*k, I] fp32
  const void *sh_src; // gate+up: x; down: act_sh [N, Is] fp32
  int src_by_token;   // routed input row = route_tok[p] (1) or p (0)
  float *out;         // gate+up: act [N*k, I]; down: y [N*k, h]
  float *sh_out;      // gate+up: act_sh [N, Is]; down: y_sh [N, h]
  const int32_t *n_active, *active, *off, *route_tok;
  int N;
  int sh_items;       // items of the shared expert (0 = none)
  int tiles;          // items per routed expert
  int max_active;     // upper bound of *n_active, min(E, N*k)
};

// fmt: 0 f32, 1 bf16, 2 fp8 e4m3 b128, 3 mxfp4; nmat: 2 = gate+up (SiLU*up
// epilogue), 1 = down; src_f32: inputs are fp32 in memory; max_items: the
// host's upper bound of the item count.
hipError_t launch_expert_gemv(int fmt, int nmat, bool src_f32, const GemvArgs &a, int max_items,
                              hipStream_t s);

struct BlendArgs {
  const float *y;        // [N*k, h]
  const float *y_sh;     // [N, h] or NULL
  const float *w;        // [N, k]
  const int32_t *route_pos;
  const void *x;         // [N, h] act dtype (for the shared gate vector)
  const void *gate_vec;  // [h] act dtype or NULL
  void *out;             // [N, h] act dtype
  int N, h, k;
};
hipError_t launch_blend(bool act_f32, const BlendArgs &a, hipStream_t s);

}  // namespace moe
