/*
 * moe_wave.h -- C ABI of the MI355X (gfx950) MoE decode-layer library.
 *
 * The library computes the mixture-of-experts layer of one decode step over
 * N token rows, as the pages describe it:
 *   - MoeLayer::forward (forward.rs): router gate GEMV -> scored top-k ->
 *     expert gate+up -> act(gate)*up -> down -> weighted-sum blend with the
 *     shared expert;
 *   - forward_token_major_decode (forward_token_major.rs): the same steps
 *     over every (token, expert-slot) route of N rows;
 *   - grouped_route (forward_fp8_grouped_router.rs): router logits and top-k
 *     indices/weights of m rows, the router read once for all rows.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a caller-owned DEVICE pointer; row-major; no
 *     padding between rows.  The library never allocates, never frees, never
 *     synchronises the stream and never branches on device data on the
 *     host, so every call can be captured into a HIP graph.
 *   - Work is enqueued on `stream` (0 = the null stream) and completes
 *     asynchronously; results are valid once the stream reaches that point.
 *   - Status: MOE_OK (0), or a negative MOE_E* code.  Every argument check
 *     happens on the host before anything is enqueued; on an error nothing is
 *     enqueued and moe_last_error() names the failing argument.
 *   - The workspace `ws` (moe_workspace_size bytes, 256-byte aligned) holds
 *     the routing, compaction and intermediate buffers of one call, and a few
 *     counters the kernels use to find the last workgroup of a pass.  It must
 *     be zero-filled once before its first use (hipMemset, torch.zeros);
 *     every call leaves those counters at zero again, so later calls need no
 *     clearing.  Calls that overlap in time must use different workspaces.
 *   - Results are deterministic: the same inputs give the same bits on every
 *     run.  How far a row's result depends on the other rows of the call:
 *       N <= 4: not at all.  A VALU router computes its logits, and every
 *         expert product runs on the VALU path, the same way whatever the
 *         other rows are.
 *       N > 4: its logits, routing indices and weights do not (a K-split
 *         MFMA router, which sums each logit in its own fixed order); its
 *         output bits do, to rounding: an expert with two or more routes in
 *         the call runs its products on MFMA, one with a single route on
 *         the VALU path.
 *     Between N <= 4 and N > 4 a row's logits agree to rounding only, so on
 *     a near tie (k-th and (k+1)-th keys within a few ulps) the two may pick
 *     different experts for the same row.  The pages' per-row router keeps a
 *     row's result independent of the grouping at any N
 *     (forward_fp8_grouped_router.rs, router_block_rows); this library gives
 *     that up above 4 rows so that the router is read once per call and
 *     grouped experts run on MFMA.
 *
 * Shapes: h = hidden, E = num_experts, k = top_k, I = inter, Is = shared_inter.
 * Limits: 1 <= N <= 4096, 1 <= k <= min(E, 32), E <= 1024, h % 32 == 0,
 * I % 32 == 0, Is % 32 == 0, h <= 16384 (h <= 8192 with fp32 activations),
 * I <= 16384, Is <= 16384.
 */
#ifndef MOE_WAVE_H
#define MOE_WAVE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: route, experts, layer (with norm and hash variants).
 * 2: adds moe_experts_forward_partial and moe_shared_combine; rejects
 *    hidden > 8192 with fp32 activations.
 * 3: adds moe_probe_stream_read and moe_layer_forward_static.
 * 4: moe_cfg gains zero_experts.
 * 5: expert weights are stored in 16-row x 64-byte tiles. */
#define MOE_ABI_VERSION 5

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL_NULL (-1)   /* a required pointer is NULL */
#define MOE_EINVAL_SHAPE (-2)  /* a size is out of range or not a multiple it must be */
#define MOE_EINVAL_TOPK (-3)   /* top_k outside [1, min(E, 32)] */
#define MOE_EINVAL_DTYPE (-4)  /* unknown dtype / scoring, or a combination not supported */
#define MOE_EINVAL_ALIGN (-5)  /* a pointer is not aligned to its access width */
#define MOE_EWORKSPACE (-6)    /* ws_bytes < moe_workspace_size(cfg, N) */
#define MOE_EHIP (-7)          /* a HIP runtime call failed (no device, launch error) */

/* dtypes */
#define MOE_DT_F32 0           /* IEEE fp32 */
#define MOE_DT_BF16 1          /* bfloat16 */
#define MOE_DT_FP8_E4M3_B128 2 /* OCP E4M3 codes (u8) + fp32 scale per 128x128 block */
#define MOE_DT_MXFP4 3         /* OCP MX: e2m1 codes, 2 per byte (element 2i in the low
                                  nibble) + e8m0 (u8) scale per 32 elements of a row */

/* scoring of the router logits (forward_token_major.rs: moe_topk_softmax_batched /
 * moe_topk_sigmoid_batched) */
#define MOE_SCORING_SOFTMAX 0  /* key = logit; w = softmax over all E, taken at the k picks */
#define MOE_SCORING_SIGMOID 1  /* key = sigmoid(logit) + bias; w = sigmoid(logit) */

/* Layer configuration (the config fields forward.rs reads: hidden_size,
 * moe_intermediate_size, shared_expert_intermediate_size, num_experts,
 * num_experts_per_tok, norm_topk_prob, routed_scaling_factor). */
typedef struct moe_cfg {
  int32_t hidden;         /* h */
  int32_t num_experts;    /* E */
  int32_t top_k;          /* k */
  int32_t inter;          /* I, intermediate width of a routed expert */
  int32_t shared_inter;   /* Is, intermediate width of the shared expert; 0 = none */
  int32_t scoring;        /* MOE_SCORING_* */
  int32_t norm_topk;      /* 1: the k weights are divided by their sum */
  float routed_scaling;   /* every routing weight is multiplied by it (1.0 = none) */
  int32_t act_dtype;      /* MOE_DT_F32 or MOE_DT_BF16: x, router W, gate vector, out */
  int32_t expert_dtype;   /* MOE_DT_F32, MOE_DT_BF16, MOE_DT_FP8_E4M3_B128, MOE_DT_MXFP4 */
  int32_t zero_experts;   /* Z >= 0 zero-computation experts (0 = none), see below */
} moe_cfg;

/* Zero-computation experts (forward.rs names a zero-expert step of the layer;
 * forward_token_major.rs refuses a router wider than num_experts, a "384-wide
 * router").  With Z = zero_experts > 0 the router has E + Z rows (W [E+Z, h],
 * corr_bias [E+Z], logits [N, E+Z]); scoring and top-k run over all E + Z
 * keys, so softmax weights share one denominator over E + Z.  A pick e in
 * [E, E + Z) is a zero expert: it reads no weights and passes its input row
 * through, adding w * x_t to the blend (x_t: the row the experts read, the
 * normed row under a pre-expert norm).  E + Z <= 1024 and
 * top_k <= min(E + Z, 32).  The expert-parallel calls and hash routing take
 * Z = 0 only (MOE_EINVAL_SHAPE otherwise). */

/* Routed expert weights: device arrays of E device pointers each (pointer
 * tables indexed by expert id, as the pages' bf16/fp8 weight_ptrs and
 * scale_ptrs).  One expert's matrices, nn.Linear [out, in] (R rows of C
 * elements):
 *   gate, up  [I, h]        down [h, I]
 *   F32 / BF16: no scales (the *_scale tables may be NULL)
 *   FP8_E4M3_B128: weights u8 [R, C]; scales fp32 [ceil(R/128), ceil(C/128)]
 *   MXFP4: weights u8 [R, C/2]; scales u8 [R, C/32]
 * Scales are row-major.  Weight bytes are stored in tiles of 16 rows x 64
 * bytes, so that one 16-byte load per lane of a wave reads a whole 1 KB tile
 * (rows of rb bytes: rb = 4C, 2C, C or C/2):
 *   row group g (rows 16 g .. 16 g + 15) is 16 rb contiguous bytes at offset
 *   16 g rb; inside it, tile column t is bytes [64 t, 64 t + 64) of the 16
 *   rows, row after row (16 x 64 bytes at offset 1024 t); when rb % 64 != 0
 *   the last tile column holds the 16 rows' last rb % 64 bytes the same way.
 *   Byte b of row r is at 16 rb (r / 16) + 1024 (b / 64) + W (r % 16) + b % 64,
 *   W = 64, or rb % 64 in the last, narrower tile column.
 * (R is a multiple of 32 and rb of 16 for every shape allowed.)  Every
 * matrix must start 16-byte aligned.  Entries of experts that no route
 * selects are never read. */
typedef struct moe_expert_tables {
  const void *const *gate;
  const void *const *up;
  const void *const *down;
  const void *const *gate_scale;
  const void *const *up_scale;
  const void *const *down_scale;
} moe_expert_tables;

/* The shared expert (same format and tiled layout as the routed experts):
 * gate, up [Is, h], down [h, Is] device pointers plus scales, and an optional gate vector
 * [h] (act dtype); weights and gate vector 16-byte aligned
 * (MOE_EINVAL_ALIGN otherwise).  With the gate vector the shared output is
 * weighted by
 * sigmoid(x . gate_vec), without it by 1 (forward.rs, the weighted-sum blend
 * beside moe_weighted_sum_blend). */
typedef struct moe_shared_expert {
  const void *gate;
  const void *up;
  const void *down;
  const void *gate_scale;
  const void *up_scale;
  const void *down_scale;
  const void *gate_vec; /* nullable */
} moe_shared_expert;

/* Number of stage events moe_layer_forward records when given an event array:
 * two per stage, when the stage's first kernel starts and when its last
 * kernel ends (hipExtLaunchKernel start / stop events, so they time the
 * kernels themselves); a NULL entry is skipped.  Pass NULL while capturing a
 * graph.  [0], [1] router + top-k + route compaction; [2], [3] expert gate+up
 * pass; [4], [5] expert down pass and blend. */
#define MOE_LAYER_EVENTS 6

/* Bytes of workspace a call with this configuration and N rows needs
 * (0 if cfg is NULL or invalid). */
size_t moe_workspace_size(const moe_cfg *cfg, int32_t n_rows);

/* Router + top-k (grouped_route / grouped_route_batched, forward_fp8_grouped_router.rs).
 *   x        [N, h]  act dtype
 *   router_w [E + Z, h]  act dtype; read once per call whatever N is
 *   corr_bias [E + Z] fp32, SIGMOID scoring only (NULL = no bias); it changes
 *            the selection only, never the weights
 *   logits   [N, E + Z] fp32 out, nullable (then kept in ws)
 *   topk_idx [N, k] int32 out: expert ids in [0, E + Z), slot 0 the largest
 *            key; equal keys go to the lowest expert id
 *   topk_w   [N, k] fp32 out: routing weights (normalised if norm_topk,
 *            then times routed_scaling)
 */
int moe_route(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *router_w,
              const float *corr_bias, float *logits, int32_t *topk_idx, float *topk_w,
              void *ws, size_t ws_bytes, hipStream_t stream);

/* Experts + blend under a given routing (the expert and blend stages of
 * forward_token_major_decode: gate+up, act(gate)*up, down, weighted sum):
 *   out[t] = sum_j topk_w[t,j] * expert_{topk_idx[t,j]}(x_t)
 *            + g_t * shared(x_t),  g_t = sigmoid(x_t . gate_vec) or 1
 *   expert(v) = down( silu(gate v) * (up v) ),  silu(z) = z * sigmoid(z)
 *   x [N, h] act dtype; out [N, h] act dtype; shared nullable (no shared expert).
 *   A topk_idx entry in [E, E + Z) is a zero expert (adds topk_w * x_t); an
 *   entry outside [0, E + Z) drops that route (it adds nothing).
 */
int moe_experts_forward(const moe_cfg *cfg, int32_t n_rows, const void *x,
                        const moe_expert_tables *experts, const moe_shared_expert *shared,
                        const int32_t *topk_idx, const float *topk_w, void *out, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* Expert parallelism, one rank's share (forward.rs, MoeLayer::forward: under
 * EP each rank's partial holds only its local experts, and the shared
 * expert is added once after the all-reduce; forward_token_major.rs: the
 * all-reduce, then residual_add or moe_batched_blend).
 *
 * moe_experts_forward_partial: this rank's routed experts only, unrounded:
 *   partial[t] = sum_j topk_w[t,j] * expert_{topk_idx[t,j]}(x_t)   fp32 [N, h]
 *   experts: this rank's table of E local experts (cfg->num_experts = E);
 *   topk_idx holds local ids, and an id outside [0, E) (another rank's
 *   expert, or -1) drops that route.  The shared expert is left out whatever
 *   cfg->shared_inter says (the workspace for cfg serves).
 * moe_shared_combine: after the caller has summed the ranks' partials
 * (fp32 [N, h], partial_sum), the shared expert once, then one rounding:
 *   out[t] = partial_sum[t] + g_t * shared(x_t)   act dtype [N, h]
 *   g_t = sigmoid(gx_t . gate_vec), or 1 without a gate vector, where gx is
 *   gate_x, or x when gate_x is NULL (with a pre-expert norm, x is the
 *   normed rows the experts read and gate_x the layer's own input, which
 *   the pages' pre_expert_norm step leaves as it is for the gate);
 *   with cfg->shared_inter == 0 (shared may be NULL): out = partial_sum, rounded.
 * For one rank holding every expert, the two calls give the bits of
 * moe_experts_forward on steps of more than one row (same fp32 operations in
 * the same order; a one-row step there takes a fused kernel).  Pointers are
 * device pointers, 16-byte aligned (topk_idx, topk_w: 4); the library keeps
 * none of them after the call. */
int moe_experts_forward_partial(const moe_cfg *cfg, int32_t n_rows, const void *x,
                                const moe_expert_tables *experts, const int32_t *topk_idx,
                                const float *topk_w, float *partial, void *ws, size_t ws_bytes,
                                hipStream_t stream);
int moe_shared_combine(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *gate_x,
                       const moe_shared_expert *shared, const float *partial_sum, void *out,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer (MoeLayer::forward at N = 1, forward_token_major_decode
 * for N rows): moe_route then moe_experts_forward.  logits, topk_idx and
 * topk_w are optional outputs (NULL = kept in ws).  stage_events, when not
 * NULL, points to MOE_LAYER_EVENTS created hipEvent_t that are recorded on
 * `stream` around the stages. */
int moe_layer_forward(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *router_w,
                      const float *corr_bias, const moe_expert_tables *experts,
                      const moe_shared_expert *shared, void *out, float *logits,
                      int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                      hipStream_t stream, hipEvent_t *stage_events);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward with
 * the library's own static workspace in place of `ws`.  It calls no
 * hipMalloc, hipFree or allocating routine.  Each GPU the library runs on
 * holds one MOE_STATIC_SCRATCH_BYTES array (a file-scope __device__ array)
 * from the library's load until the process ends; its address is looked up
 * once per device with that device current.  A configuration whose
 * moe_workspace_size(cfg, n_rows) exceeds MOE_STATIC_SCRATCH_BYTES returns
 * MOE_EWORKSPACE with nothing enqueued (the MXFP4 verify layer at 256 rows
 * needs 57.8 MiB).  The first call on a device also enqueues one small
 * kernel that clears the array's counters; every call leaves them at zero.
 * All calls on one GPU share the array and keep the last call's contents:
 * calls that overlap in time on one GPU (two streams, two host threads)
 * race and give undefined results; serialise them.  Other arguments, the
 * results and their bits are those of moe_layer_forward. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_static(const moe_cfg *cfg, int32_t n_rows, const void *x,
                             const void *router_w, const float *corr_bias,
                             const moe_expert_tables *experts, const moe_shared_expert *shared,
                             void *out, float *logits, int32_t *topk_idx, float *topk_w,
                             hipStream_t stream, hipEvent_t *stage_events);

/* The layer with its optional pre-norms (forward.rs: the router reads its
 * input through the layer's router pre-norm, and the pre_expert_norm step
 * normalises the experts' input after routing, leaving the layer input for
 * the shared-expert gate):
 *   xr = rmsnorm(x, router_norm_w)  if router_norm_w, else x   (router input)
 *   xe = rmsnorm(x, expert_norm_w)  if expert_norm_w, else x   (routed and
 *                                                              shared experts)
 *   g_t = sigmoid(x_t . gate_vec): the gate reads x itself
 *   rmsnorm(x, w)[t,i] = x[t,i] * w[i] / sqrt(mean_i x[t,i]^2 + eps), in
 *   fp32, stored in the act dtype before the router and experts read it.
 *   router_norm_w, expert_norm_w: [h] act dtype, nullable, 16-byte aligned
 *   (MOE_EINVAL_ALIGN otherwise); eps in [0, 1] (MOE_EINVAL_SHAPE otherwise).  The normed rows live
 *   in ws.  With both weights NULL this is moe_layer_forward.  The norm's
 *   kernel counts in the first stage's events.  Other arguments as
 *   moe_layer_forward. */
int moe_layer_forward_norm(const moe_cfg *cfg, int32_t n_rows, const void *x,
                           const void *router_norm_w, const void *expert_norm_w, float eps,
                           const void *router_w, const float *corr_bias,
                           const moe_expert_tables *experts, const moe_shared_expert *shared,
                           void *out, float *logits, int32_t *topk_idx, float *topk_w, void *ws,
                           size_t ws_bytes, hipStream_t stream, hipEvent_t *stage_events);

/* The layer with hash routing in place of top-k (forward.rs, the
 * hash-routing branch of the top-k step): the router still computes the
 * logits, but row t's experts are the table row tid2eid[token_ids[t]], and
 *   w[t,j] = s_j / sum_j s_j (norm_topk) or s_j, times routed_scaling,
 *   s_j = sqrt(softplus(logits[t, e_j])),  softplus(z) = log(1 + e^z).
 *   token_ids [N] int32, tid2eid [vocab, k] int32 (device, 4-byte aligned).
 *   A table entry outside [0, E) drops that route (weight 0, excluded from
 *   the sum); a token id outside [0, vocab) drops the row's routes (ids -1).
 *   cfg->scoring is not used.  Other arguments as moe_layer_forward (no
 *   correction bias). */
int moe_layer_forward_hash(const moe_cfg *cfg, int32_t n_rows, const void *x,
                           const int32_t *token_ids, const int32_t *tid2eid, int32_t vocab,
                           const void *router_w, const moe_expert_tables *experts,
                           const moe_shared_expert *shared, void *out, float *logits,
                           int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t *stage_events);

/* Measurement aid, not a step of the layer: one kernel that only reads
 * `bytes` of `buf` with 128-bit loads, `grid` workgroups of 256 threads
 * striding over it, the practical streaming-read ceiling the expert passes
 * are measured beside.  buf: device, 16-byte aligned, bytes % 16 == 0,
 * zero-filled (then nothing is written); sink: device, grid * 256 uint32
 * (written only for buffers of other contents).  ev0 / ev1 (nullable) are
 * recorded when the kernel starts and ends.  MOE_EINVAL_NULL / _ALIGN /
 * _SHAPE (grid outside [1, 65536]) or MOE_EHIP on a launch error. */
int moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t grid,
                          hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

/* Static text of a status code. */
const char *moe_strerror(int code);

/* Detail of the last error on the calling thread ("" if none). */
const char *moe_last_error(void);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_WAVE_H */
