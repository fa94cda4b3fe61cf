// Host-side launchers of the MoE decode-layer kernels (internal interface
// between the C ABI in abi.hip and the kernel files).
#pragma once

#include <hip/hip_ext.h>
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
  int32_t *hist;      // multi-workgroup compaction: [Er][hist_stride(N)] route
                      // counts per (expert, group of 16 rows), then prefixes
};

// Steps of more than this many 16-row groups compact their routes with every
// top-k workgroup taking part (histogram, scan, scatter); smaller ones in the
// top-k launch's last workgroup alone.
constexpr int PAR_COMPACT_MIN_GROUPS = 8;
// row stride (int32 entries) of Compact::hist for N rows: the 16-row groups,
// rounded up to 4 for 16-byte loads
constexpr int hist_stride(int N) { return (((N + 15) / 16) + 3) & ~3; }

// Up to this many rows a VALU router runs and its last workgroup also does
// top-k and compaction (one launch); above it a K-split MFMA router writes
// partial logits and a multi-workgroup top-k kernel follows.
constexpr int FUSE_MAX_N = 4;

struct RouteLaunch {
  const void *x;        // [N, h] act dtype
  const void *W;        // [E, h] act dtype (router weights), used if do_router
  float *logits;        // [N, E]
  int N, E, h, act_f32; // E: router width, the Er real experts then the zero experts
  int Er;               // real experts (ids >= Er are zero experts: no route)
  const float *bias;    // [E] or NULL (sigmoid scoring)
  int32_t *idx;         // [N, k]
  float *w;             // [N, k]
  int k, scoring, norm;
  float rsf;
  int do_router, do_topk, do_compact;
  Compact c;
  uint32_t *counter;    // zeroed workspace word, left at zero
  const void *gate_vec; // shared-expert gate vector or NULL
  const void *gx;       // [N, h] rows the gate vector reads (NULL: x)
  const int32_t *token_ids;  // hash routing instead of top-k: [N] token ids (NULL: top-k)
  const int32_t *tid2eid;    // [vocab, k] expert ids per token
  int vocab;
  float *g;             // [N] sigmoid(gx_t . gate_vec)
  float *part;          // [S][N][E] router partials (N > FUSE_MAX_N, bf16)
  // pre-norms inside the router (only where router_norms_fused holds): the
  // router's and the experts' RMSNorm weights [h] (act dtype, nullable; the
  // router then reads x normed with wr), the experts' normed rows out [N, h]
  const void *wr, *we;
  void *xe;
  float eps;
};

// whether launch_route can compute the pre-norms inside the router
bool router_norms_fused(int N, int h, bool act_f32);

// hidden columns per K slice of the N > FUSE_MAX_N router
int router_kslice(int h, int E);
// ev0 / ev1 (nullable): recorded when the stage's first kernel starts and its
// last kernel ends (hipExtLaunchKernel start / stop events).
hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

// The layer's pre-norms: RMSNorm of the N input rows with the router's
// weights into xr and with the experts' weights into xe (a NULL weight vector
// skips its output).
struct NormArgs {
  const void *x;         // [N, h] act dtype
  const void *wr, *we;   // [h] act dtype, nullable
  void *xr, *xe;         // [N, h] act dtype
  int N, h;
  float eps;
};

hipError_t launch_rmsnorm(bool act_f32, const NormArgs &a, hipStream_t s, hipEvent_t ev0,
                          hipEvent_t ev1);

// One streaming pass over the active experts (and the shared expert).
struct GemvArgs {
  const void *const *w0;  // routed weight tables [E]: gate (gate+up pass) or down
  const void *const *w1;  // up (gate+up pass) or NULL
  const void *const *s0;  // scale tables or NULL
  const void *const *s1;
  const void *sh_w0, *sh_w1, *sh_s0, *sh_s1;  // shared expert (sh_w0 NULL = none)
  int rows, K;        // routed matrix: rows x K
  int sh_rows, sh_K;  // shared matrix
  const void *src;    // gate+up: x [N, h] (act dtype); down: act [N*k, I] (bf16; fp32 experts: fp32)
  const void *sh_src; // gate+up: x; down: act_sh [N, Is], likewise
  int src_by_token;   // routed input row = route_tok[p] (1) or p (0)
  const int32_t *out_map;  // routed output row = out_map[p], or p if NULL
  void *out;          // gate+up: act [N*k, I] by position p; down: y [N*k, h] fp32 by route t*k+j
  void *sh_out;       // gate+up: act_sh [N, Is]; down: y_sh [N, h] fp32
  const int32_t *n_active, *active, *off, *route_tok;
  int N;
  int sh_tiles;       // tiles of the shared matrix (0 = no shared expert)
  int sh_chunk;       // shared-expert routes per item (set by launch_expert_gemv)
  int sh_items;       // items of the shared expert: tiles x route chunks (likewise)
  int tiles;          // items per routed expert
  int max_active;     // upper bound of *n_active, min(E, N*k)
  int E;              // experts (entries of the weight tables)
  int lds_bytes;      // dynamic LDS of the launch (set by launch_expert_gemv)
  int max_r;          // most routes an expert can have in this launch (set likewise)
  int gemm;           // grouped-GEMM mode beside the MFMA path (set likewise)
  int npass;          // passes of tr rows per routed item (set likewise; items cover tr npass rows)
  int sh_npass;       // passes of tr rows per shared-expert item (set likewise)
  int tail_e;         // the last tail_e active experts take one-tile items (set likewise)
};

// The weighted blend of the routed outputs and the shared expert.
struct BlendArgs {
  const float *y;           // [N*k, h], row t*k + j
  const float *y_sh;        // [N, h] or NULL
  const float *w;           // [N, k]
  const float *g;           // [N] shared-expert gate values or NULL (= 1)
  const int32_t *route_pos; // [N*k]: < 0 for a dropped route
  const float *base;        // [N, h] fp32 added first, or NULL
  void *out;                // [N, h] act dtype (fp32 when launched with out_f32)
  int N, h, k;              // k = 0: no routes (base and the shared expert only)
  // zero-computation experts (Z > 0): a slot whose id is in [E, E + Z) adds
  // w * x[t] (x: the experts' input rows, act dtype)
  const int32_t *idx;       // [N, k] expert ids
  const void *x;            // [N, h]
  int E, Z, x_f32;
};

// weight rows per item (64 or 16) for a rows x K matrix and this many active
// experts at most: the largest tile that gives at least min_items items
int expert_tile_rows(int K, int rows, int max_active, int min_items);

// Shared-expert routes per item beside the MFMA path: one route group (the
// grouped-GEMM form's groups are 64 routes wide).
constexpr int SH_CHUNK_MIXED = 16;
constexpr int SH_CHUNK_GEMM = 64;
// Workgroups per CU of the expert pass beside the MFMA path: 3 for the down
// pass (its LDS is sized to match), 2 for gate+up (measured on MI355X).
constexpr int mixed_blocks_per_cu(int nmat) { return nmat == 1 ? 3 : 2; }
// The grouped-GEMM form's items: gemm_mr 128-row tiles, computed together
// (each wave holds a 16-row group of every tile); the down pass (one
// matrix) has the registers for 4 a wave, gate+up for 2
constexpr int GEMM_MR = 2;
constexpr int gemm_mr(int fmt, int nmat) { return nmat == 1 ? 4 : GEMM_MR; }

// nmat: 2 = gate+up (SiLU*up epilogue, inputs x in the act dtype), 1 = down
// (fp32 act inputs); max_items: the host's upper bound of the routed items;
// tr: rows per item; max_r: the most routes any expert can have (N for a
// top-k routing, N*k for a caller's).  The act dtype is fp32 exactly when the
// experts are fp32.
// wide: the experts average 32 or more routes (a large step): experts of two
// or more routes then take the grouped-GEMM form of the MFMA path.
// (a.tiles and a.sh_tiles count tiles of tr rows; the launch groups them
// into items of npass tiles where the MFMA path gains by it)
hipError_t launch_expert_gemv(int fmt, int nmat, const GemvArgs &a, int max_items, int tr,
                              int max_r, bool wide, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1);

hipError_t launch_blend(bool act_f32, const BlendArgs &a, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1);

// The down pass and the blend of a one-row step in one kernel (routed and
// shared K equal): workgroup b owns output columns [b tr, b tr + tr).
struct Down1Args {
  const void *const *w;      // routed down tables [E]
  const void *const *s;      // their scale tables or NULL
  const void *sh_w, *sh_s;   // shared down matrix and scales (sh_w NULL = none)
  int h, K, tr;              // down matrices h x K; output columns per workgroup (4)
  const void *act;           // act [k, K] by route position (bf16; fp32 for fp32 experts)
  const void *act_sh;        // act_sh [1, K]
  const int32_t *idx;        // [k] expert of each slot
  const int32_t *route_pos;  // [k] act position of each slot (-1: dropped)
  const float *w_slot;       // [k] slot weights
  const float *g;            // [1] shared-expert gate value or NULL (= 1)
  void *out;                 // [1, h] act dtype
  int k;
  const void *x;             // [1, h] the experts' input row (act dtype)
  int E, Z;                  // a slot with an id in [E, E + Z) adds w * x
};

// whether a one-row step takes down_blend1 (and its launch shape); returns
// false where the two-kernel form serves better
bool down_blend1_plan(int fmt, int N, int h, int K, int sh_K, bool has_sh, int k, int *tr,
                      int *lds_bytes);
hipError_t launch_down_blend1(int fmt, const Down1Args &a, int lds_bytes, hipStream_t s,
                              hipEvent_t ev0, hipEvent_t ev1);

}  // namespace moe
