// C ABI of the MoE decode-layer library: argument checks, workspace layout
// and the launch sequence router -> top-k + compaction -> gate+up -> down ->
// blend, all on the caller's stream with no host synchronisation.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_wave.h"
#include "launch.h"

using namespace moe;

// The workspace of moe_layer_forward_static, for callers that cannot
// allocate: one copy per GPU, held from the library's load until the process
// ends.  Host code never uses this name as an address: the per-device
// address comes from hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

// zeroes n words (the workspace's counters before their first use)
__global__ void zero_words_kernel(uint32_t *p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

constexpr int MAX_N = 4096;
constexpr int MAX_E = 1024;
constexpr int MAX_K = 32;
constexpr int MAX_DIM = 16384;
constexpr int MAX_DIM_F32 = 8192;  // hidden with fp32 activations

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t counter, logits, part, idx, w, g, n_active, active, off, route_tok, route_src,
      route_pos, hist, act, act_sh, y, y_sh, xr, xe, total;
};

Layout layout(const moe_cfg &c, int N) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align256(o + bytes);
    return r;
  };
  const size_t NK = (size_t)N * c.top_k;
  const size_t maxa = NK < (size_t)c.num_experts ? NK : (size_t)c.num_experts;
  const size_t EW = (size_t)c.num_experts + c.zero_experts;  // router width
  L.counter = take(4);                          // zero at rest
  L.logits = take((size_t)N * EW * 4);
  {
    const int KS = router_kslice(c.hidden, (int)EW);
    const size_t S = (c.hidden + KS - 1) / KS;
    L.part = take(N > FUSE_MAX_N ? S * N * EW * 4 : 0);
  }
  L.idx = take(NK * 4);
  L.w = take(NK * 4);
  L.g = take((size_t)N * 4);
  L.n_active = take(4);
  L.active = take(maxa * 4);
  L.off = take((maxa + 1) * 4);
  L.route_tok = take(NK * 4);
  L.route_src = take(NK * 4);
  L.route_pos = take(NK * 4);
  L.hist = take(N > FUSE_MAX_N ? (size_t)c.num_experts * hist_stride(N) * 4 : 0);
  L.act = take(NK * c.inter * 4);  // fp32 for fp32 experts, else bf16 in the first half
  L.act_sh = take((size_t)N * c.shared_inter * 4);
  L.y = take(NK * c.hidden * 4);
  L.y_sh = take(c.shared_inter > 0 ? (size_t)N * c.hidden * 4 : 0);
  // the pre-normed rows of moe_layer_forward_norm (router's, experts')
  const size_t ab = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  L.xr = take((size_t)N * c.hidden * ab);
  L.xe = take((size_t)N * c.hidden * ab);
  L.total = o;
  return L;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_cfg(const moe_cfg *c, int N) {
  if (!c) return fail(MOE_EINVAL_NULL, "cfg is NULL");
  if (N < 1 || N > MAX_N) return fail(MOE_EINVAL_SHAPE, "n_rows=%d outside [1, %d]", N, MAX_N);
  if (c->num_experts < 1 || c->num_experts > MAX_E)
    return fail(MOE_EINVAL_SHAPE, "num_experts=%d outside [1, %d]", c->num_experts, MAX_E);
  if (c->zero_experts < 0 || c->zero_experts > MAX_E - c->num_experts)
    return fail(MOE_EINVAL_SHAPE, "zero_experts=%d outside [0, %d - num_experts]",
                c->zero_experts, MAX_E);
  if (c->top_k < 1 || c->top_k > c->num_experts + c->zero_experts || c->top_k > MAX_K)
    return fail(MOE_EINVAL_TOPK, "top_k=%d outside [1, min(num_experts + zero_experts=%d, %d)]",
                c->top_k, c->num_experts + c->zero_experts, MAX_K);
  if (c->hidden < 32 || c->hidden > MAX_DIM || c->hidden % 32)
    return fail(MOE_EINVAL_SHAPE, "hidden=%d must be a multiple of 32 in [32, %d]", c->hidden,
                MAX_DIM);
  if (c->inter < 32 || c->inter > MAX_DIM || c->inter % 32)
    return fail(MOE_EINVAL_SHAPE, "inter=%d must be a multiple of 32 in [32, %d]", c->inter,
                MAX_DIM);
  if (c->shared_inter < 0 || c->shared_inter > MAX_DIM || c->shared_inter % 32)
    return fail(MOE_EINVAL_SHAPE, "shared_inter=%d must be 0 or a multiple of 32 <= %d",
                c->shared_inter, MAX_DIM);
  if (c->scoring != MOE_SCORING_SOFTMAX && c->scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_EINVAL_DTYPE, "unknown scoring %d", c->scoring);
  if (c->norm_topk != 0 && c->norm_topk != 1)
    return fail(MOE_EINVAL_SHAPE, "norm_topk=%d must be 0 or 1", c->norm_topk);
  if (!(c->routed_scaling == c->routed_scaling) || c->routed_scaling == 1.0f / 0.0f ||
      c->routed_scaling == -1.0f / 0.0f)
    return fail(MOE_EINVAL_SHAPE, "routed_scaling must be finite");
  const bool f32 = c->act_dtype == MOE_DT_F32 && c->expert_dtype == MOE_DT_F32;
  const bool bf = c->act_dtype == MOE_DT_BF16 &&
                  (c->expert_dtype == MOE_DT_BF16 || c->expert_dtype == MOE_DT_FP8_E4M3_B128 ||
                   c->expert_dtype == MOE_DT_MXFP4);
  if (!f32 && !bf)
    return fail(MOE_EINVAL_DTYPE,
                "unsupported dtypes act=%d expert=%d (fp32/fp32 or bf16 with bf16, fp8 or "
                "mxfp4 experts)",
                c->act_dtype, c->expert_dtype);
  // the router holds at most 8 16-byte chunks of a quarter row per lane: 8192
  // fp32 or 16384 bf16 values
  if (f32 && c->hidden > MAX_DIM_F32)
    return fail(MOE_EINVAL_SHAPE, "hidden=%d above %d with fp32 activations", c->hidden,
                MAX_DIM_F32);
  return MOE_OK;
}

int check_ws(const moe_cfg *c, int N, void *ws, size_t ws_bytes, Layout *L) {
  *L = layout(*c, N);
  if (!ws) return fail(MOE_EINVAL_NULL, "ws is NULL");
  if (!aligned(ws, 256)) return fail(MOE_EINVAL_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < L->total)
    return fail(MOE_EWORKSPACE, "ws_bytes=%zu < required %zu", ws_bytes, L->total);
  return MOE_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
  return (T *)((char *)ws + off);
}

Compact compact_of(void *ws, const Layout &L) {
  return Compact{at<int32_t>(ws, L.n_active), at<int32_t>(ws, L.active), at<int32_t>(ws, L.off),
                 at<int32_t>(ws, L.route_tok), at<int32_t>(ws, L.route_src),
                 at<int32_t>(ws, L.route_pos), at<int32_t>(ws, L.hist)};
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_route_args(const moe_cfg *c, const void *x, const void *router_w, const float *bias,
                     const float *logits, const int32_t *idx, const float *w) {
  if (!x) return fail(MOE_EINVAL_NULL, "x is NULL");
  if (!router_w) return fail(MOE_EINVAL_NULL, "router_w is NULL");
  if (!idx) return fail(MOE_EINVAL_NULL, "topk_idx is NULL");
  if (!w) return fail(MOE_EINVAL_NULL, "topk_w is NULL");
  if (!aligned(x, 16) || !aligned(router_w, 16))
    return fail(MOE_EINVAL_ALIGN, "x and router_w must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4)) ||
      (bias && !aligned(bias, 4)))
    return fail(MOE_EINVAL_ALIGN, "logits, bias, topk_idx and topk_w must be 4-byte aligned");
  if (bias && c->scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_EINVAL_DTYPE, "corr_bias needs SIGMOID scoring");
  return MOE_OK;
}

bool scaled_fmt(const moe_cfg *c) {
  return c->expert_dtype == MOE_DT_FP8_E4M3_B128 || c->expert_dtype == MOE_DT_MXFP4;
}

int check_shared_args(const moe_cfg *c, const moe_shared_expert *sh) {
  const bool scaled = scaled_fmt(c);
  if (c->shared_inter > 0) {
    if (!sh) return fail(MOE_EINVAL_NULL, "shared_inter > 0 but shared is NULL");
    if (!sh->gate || !sh->up || !sh->down)
      return fail(MOE_EINVAL_NULL, "shared expert weight is NULL");
    if (scaled && (!sh->gate_scale || !sh->up_scale || !sh->down_scale))
      return fail(MOE_EINVAL_NULL, "shared expert scale is NULL for a scaled format");
    if (!aligned(sh->gate, 16) || !aligned(sh->up, 16) || !aligned(sh->down, 16) ||
        !aligned(sh->gate_vec, 16))
      return fail(MOE_EINVAL_ALIGN, "shared expert weights and gate vector must be 16-byte aligned");
  }
  return MOE_OK;
}

int check_expert_args(const moe_cfg *c, const void *x, const moe_expert_tables *t,
                      const moe_shared_expert *sh, const void *out) {
  if (!x) return fail(MOE_EINVAL_NULL, "x is NULL");
  if (!out) return fail(MOE_EINVAL_NULL, "out is NULL");
  if (!t) return fail(MOE_EINVAL_NULL, "experts is NULL");
  if (!t->gate || !t->up || !t->down) return fail(MOE_EINVAL_NULL, "expert weight table is NULL");
  if (scaled_fmt(c) && (!t->gate_scale || !t->up_scale || !t->down_scale))
    return fail(MOE_EINVAL_NULL, "expert scale table is NULL for a scaled format");
  if (!aligned(x, 16) || !aligned(out, 16))
    return fail(MOE_EINVAL_ALIGN, "x and out must be 16-byte aligned");
  return check_shared_args(c, sh);
}

int fmt_of(int expert_dtype) { return expert_dtype; }  // same numbering as moe::Fmt

// Stage event i of the caller's array, or NULL.
hipEvent_t evi(hipEvent_t *ev, int i) { return ev ? ev[i] : nullptr; }

// What run_experts computes: the layer's expert stages; an expert-parallel
// rank's fp32 partial (routed experts only, c without a shared expert); or
// the combine after the all-reduce (the shared expert only, added to a base).
enum RunMode { RUN_LAYER, RUN_PARTIAL, RUN_COMBINE };

// the expert stages, given compacted routes in ws (RUN_COMBINE: none are read)
int run_experts(const moe_cfg *c, int N, const void *x, const moe_expert_tables *t,
                const moe_shared_expert *sh, const int32_t *idx, const float *w, void *out,
                void *ws, const Layout &L, hipStream_t s, hipEvent_t *ev, int max_r,
                RunMode mode = RUN_LAYER, const float *base = nullptr) {
  const bool has_sh = c->shared_inter > 0;
  const int NK = N * c->top_k;
  // tiles and kernel forms as the layer picks them, so that the shared
  // expert's items compute the same bits in every mode; RUN_COMBINE then
  // allows no routed item (the kernels bound their item loop by max_active)
  const int maxa_layer = NK < c->num_experts ? NK : c->num_experts;
  const int maxa = mode == RUN_COMBINE ? 0 : maxa_layer;
  const int fmt = fmt_of(c->expert_dtype);
  hipError_t e;

  GemvArgs g{};
  if (t) {
    g.w0 = t->gate;
    g.w1 = t->up;
    g.s0 = t->gate_scale;
    g.s1 = t->up_scale;
  }
  if (has_sh) {
    g.sh_w0 = sh->gate;
    g.sh_w1 = sh->up;
    g.sh_s0 = sh->gate_scale;
    g.sh_s1 = sh->up_scale;
  }
  g.rows = c->inter;
  g.K = c->hidden;
  g.sh_rows = c->shared_inter;
  g.sh_K = c->hidden;
  g.src = x;
  g.sh_src = x;
  g.src_by_token = 1;
  g.out = at<void>(ws, L.act);
  g.sh_out = at<void>(ws, L.act_sh);
  g.n_active = at<int32_t>(ws, L.n_active);
  g.active = at<int32_t>(ws, L.active);
  g.off = at<int32_t>(ws, L.off);
  g.route_tok = at<int32_t>(ws, L.route_tok);
  g.N = N;
  // Item counts measured best on MI355X: 2 per CU, except a gate+up pass
  // whose experts have at most 4 routes each (VALU path only), which streams
  // best in 8 items per CU.
  const int tr_gu = expert_tile_rows(c->hidden, c->inter, maxa_layer, max_r <= 4 ? 2048 : 512);
  g.tiles = (c->inter + tr_gu - 1) / tr_gu;
  g.sh_tiles = has_sh ? (c->shared_inter + tr_gu - 1) / tr_gu : 0;
  g.max_active = maxa;
  g.E = c->num_experts;
  // a large step: the experts average 32 or more routes
  const bool wide = (long)NK >= 32L * c->num_experts;
  // the expert passes have work unless a combine has no shared expert
  const bool passes = mode != RUN_COMBINE || has_sh;
  if (passes && (e = launch_expert_gemv(fmt, 2, g, maxa * g.tiles, tr_gu, max_r, wide, s,
                                        evi(ev, 2), evi(ev, 3))) != hipSuccess)
    return hip_fail(e, "gate+up launch");

  GemvArgs d{};
  if (t) {
    d.w0 = t->down;
    d.s0 = t->down_scale;
  }
  if (has_sh) {
    d.sh_w0 = sh->down;
    d.sh_s0 = sh->down_scale;
  }
  d.rows = c->hidden;
  d.K = c->inter;
  d.sh_rows = c->hidden;
  d.sh_K = c->shared_inter;
  d.src = at<void>(ws, L.act);
  d.sh_src = at<void>(ws, L.act_sh);
  d.src_by_token = 0;
  d.out_map = at<int32_t>(ws, L.route_src);  // y rows in (token, slot) order
  d.out = at<float>(ws, L.y);
  d.sh_out = at<float>(ws, L.y_sh);
  d.n_active = g.n_active;
  d.active = g.active;
  d.off = g.off;
  d.route_tok = g.route_tok;
  d.N = N;
  const int tr_dn = expert_tile_rows(c->inter, c->hidden, maxa_layer, 512);
  d.tiles = (c->hidden + tr_dn - 1) / tr_dn;
  d.sh_tiles = has_sh ? d.tiles : 0;
  d.max_active = maxa;
  d.E = c->num_experts;

  BlendArgs b{};
  b.y = at<float>(ws, L.y);
  b.y_sh = has_sh ? at<float>(ws, L.y_sh) : nullptr;
  b.w = w;
  b.g = (has_sh && sh->gate_vec) ? at<float>(ws, L.g) : nullptr;
  b.route_pos = at<int32_t>(ws, L.route_pos);
  b.base = base;
  b.out = out;
  b.N = N;
  b.h = c->hidden;
  b.k = mode == RUN_COMBINE ? 0 : c->top_k;
  b.idx = idx;
  b.x = x;
  b.E = c->num_experts;
  b.Z = mode == RUN_LAYER ? c->zero_experts : 0;
  b.x_f32 = c->act_dtype == MOE_DT_F32;
  // a one-row step whose down pass streams few bytes: down and blend in one kernel
  int tr1 = 0, lds1 = 0;
  if (mode == RUN_LAYER && down_blend1_plan(fmt, N, c->hidden, c->inter, c->shared_inter, has_sh,
                                            c->top_k, &tr1, &lds1)) {
    Down1Args o{};
    o.w = t->down;
    o.s = t->down_scale;
    o.sh_w = has_sh ? sh->down : nullptr;
    o.sh_s = has_sh ? sh->down_scale : nullptr;
    o.h = c->hidden;
    o.K = c->inter;
    o.tr = tr1;
    o.act = at<void>(ws, L.act);
    o.act_sh = at<void>(ws, L.act_sh);
    o.idx = idx;
    o.route_pos = b.route_pos;
    o.w_slot = w;
    o.g = b.g;
    o.out = out;
    o.k = c->top_k;
    o.x = x;
    o.E = c->num_experts;
    o.Z = c->zero_experts;
    if ((e = launch_down_blend1(fmt, o, lds1, s, evi(ev, 4), evi(ev, 5))) != hipSuccess)
      return hip_fail(e, "down+blend launch");
    return MOE_OK;
  }
  if (passes && (e = launch_expert_gemv(fmt, 1, d, maxa * d.tiles, tr_dn, max_r, wide, s,
                                        evi(ev, 4), nullptr)) != hipSuccess)
    return hip_fail(e, "down launch");
  const bool out_f32 = mode == RUN_PARTIAL || c->act_dtype == MOE_DT_F32;
  if ((e = launch_blend(out_f32, b, s, nullptr, evi(ev, 5))) != hipSuccess)
    return hip_fail(e, "blend launch");
  return MOE_OK;
}

// Per device: the address of `scratch` and whether its counters have been
// cleared.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];
bool g_scratch_clear[MAX_DEVICES];

// The current device's static scratch address (looked up once per device,
// with that device current; nothing is enqueued).
int static_scratch(void **out, int *dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(MOE_EHIP, "device %d outside the %d the static scratch serves", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256) return fail(MOE_EHIP, "static scratch address %p", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  *dev_out = dev;
  return MOE_OK;
}

// Before the first use on a device the counters at the workspace's start
// are cleared by a kernel on the caller's stream (a kernel, not a memset, so
// a graph capturing this call replays it correctly); every call leaves them
// at zero after that.
int clear_static_counters(void *p, int dev, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_clear[dev]) return MOE_OK;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, s, (uint32_t *)p, 64);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "static scratch clearing launch");
  g_scratch_clear[dev] = true;
  return MOE_OK;
}

RouteLaunch route_launch(const moe_cfg *c, int N, const void *x, const void *router_w,
                         const float *bias, float *logits, int32_t *idx, float *w, void *ws,
                         const Layout &L, const moe_shared_expert *sh) {
  RouteLaunch r{};
  r.x = x;
  r.W = router_w;
  r.logits = logits;
  r.N = N;
  r.E = c->num_experts + c->zero_experts;
  r.Er = c->num_experts;
  r.h = c->hidden;
  r.act_f32 = c->act_dtype == MOE_DT_F32;
  r.bias = bias;
  r.idx = idx;
  r.w = w;
  r.k = c->top_k;
  r.scoring = c->scoring;
  r.norm = c->norm_topk;
  r.rsf = c->routed_scaling;
  r.c = compact_of(ws, L);
  r.counter = at<uint32_t>(ws, L.counter);
  r.gate_vec = (c->shared_inter > 0 && sh) ? sh->gate_vec : nullptr;
  r.g = at<float>(ws, L.g);
  r.part = at<float>(ws, L.part);
  return r;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_cfg *cfg, int32_t n_rows) {
  if (check_cfg(cfg, n_rows) != MOE_OK) return 0;
  return layout(*cfg, n_rows).total;
}

int moe_route(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *router_w,
              const float *corr_bias, float *logits, int32_t *topk_idx, float *topk_w, void *ws,
              size_t ws_bytes, hipStream_t stream) {
  int rc;
  Layout L;
  if ((rc = check_cfg(cfg, n_rows)) || (rc = check_ws(cfg, n_rows, ws, ws_bytes, &L)) ||
      (rc = check_route_args(cfg, x, router_w, corr_bias, logits, topk_idx, topk_w)))
    return rc;
  float *lg = logits ? logits : at<float>(ws, L.logits);
  RouteLaunch r = route_launch(cfg, n_rows, x, router_w, corr_bias, lg, topk_idx, topk_w, ws, L,
                               nullptr);
  r.do_router = 1;
  r.do_topk = 1;
  r.do_compact = 0;
  hipError_t e;
  if ((e = launch_route(r, stream, nullptr, nullptr)) != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

int moe_experts_forward(const moe_cfg *cfg, int32_t n_rows, const void *x,
                        const moe_expert_tables *experts, const moe_shared_expert *shared,
                        const int32_t *topk_idx, const float *topk_w, void *out, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
  int rc;
  Layout L;
  if ((rc = check_cfg(cfg, n_rows)) || (rc = check_ws(cfg, n_rows, ws, ws_bytes, &L)) ||
      (rc = check_expert_args(cfg, x, experts, shared, out)))
    return rc;
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL_NULL, "topk_idx / topk_w is NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4))
    return fail(MOE_EINVAL_ALIGN, "topk_idx and topk_w must be 4-byte aligned");
  RouteLaunch r = route_launch(cfg, n_rows, x, nullptr, nullptr, nullptr,
                               const_cast<int32_t *>(topk_idx), nullptr, ws, L, shared);
  r.do_router = 0;
  r.do_topk = 0;
  r.do_compact = 1;
  hipError_t e;
  if ((e = launch_route(r, stream, nullptr, nullptr)) != hipSuccess)
    return hip_fail(e, "compaction launch");
  // a caller's routing may repeat an expert within a row
  if ((rc = run_experts(cfg, n_rows, x, experts, shared, topk_idx, topk_w, out, ws, L, stream,
                        nullptr, n_rows * cfg->top_k)))
    return rc;
  return ok();
}

int moe_experts_forward_partial(const moe_cfg *cfg, int32_t n_rows, const void *x,
                                const moe_expert_tables *experts, const int32_t *topk_idx,
                                const float *topk_w, float *partial, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  int rc;
  if ((rc = check_cfg(cfg, n_rows))) return rc;
  if (cfg->zero_experts)
    return fail(MOE_EINVAL_SHAPE, "the expert-parallel calls take no zero experts");
  moe_cfg c = *cfg;  // the shared expert is left out of a partial
  c.shared_inter = 0;
  Layout L;
  if ((rc = check_ws(&c, n_rows, ws, ws_bytes, &L)) ||
      (rc = check_expert_args(&c, x, experts, nullptr, partial)))
    return rc;
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL_NULL, "topk_idx / topk_w is NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4))
    return fail(MOE_EINVAL_ALIGN, "topk_idx and topk_w must be 4-byte aligned");
  RouteLaunch r = route_launch(&c, n_rows, x, nullptr, nullptr, nullptr,
                               const_cast<int32_t *>(topk_idx), nullptr, ws, L, nullptr);
  r.do_router = 0;
  r.do_topk = 0;
  r.do_compact = 1;
  hipError_t e;
  if ((e = launch_route(r, stream, nullptr, nullptr)) != hipSuccess)
    return hip_fail(e, "compaction launch");
  if ((rc = run_experts(&c, n_rows, x, experts, nullptr, topk_idx, topk_w, partial, ws, L, stream,
                        nullptr, n_rows * c.top_k, RUN_PARTIAL)))
    return rc;
  return ok();
}

int moe_shared_combine(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *gate_x,
                       const moe_shared_expert *shared, const float *partial_sum, void *out,
                       void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc;
  Layout L;
  if ((rc = check_cfg(cfg, n_rows)) || (rc = check_ws(cfg, n_rows, ws, ws_bytes, &L)) ||
      (rc = check_shared_args(cfg, shared)))
    return rc;
  if (cfg->zero_experts)
    return fail(MOE_EINVAL_SHAPE, "the expert-parallel calls take no zero experts");
  if (!x || !partial_sum || !out) return fail(MOE_EINVAL_NULL, "x / partial_sum / out is NULL");
  if (!aligned(x, 16) || !aligned(partial_sum, 16) || !aligned(out, 16) || !aligned(gate_x, 16))
    return fail(MOE_EINVAL_ALIGN, "x, gate_x, partial_sum and out must be 16-byte aligned");
  hipError_t e;
  const bool has_sh = cfg->shared_inter > 0;
  if (has_sh && shared->gate_vec) {  // g_t = sigmoid(gate_x_t . gate_vec)
    RouteLaunch r = route_launch(cfg, n_rows, x, nullptr, nullptr, nullptr, nullptr, nullptr, ws,
                                 L, shared);
    r.gx = gate_x ? gate_x : x;
    r.do_router = 0;
    r.do_topk = 0;
    r.do_compact = 0;
    if ((e = launch_route(r, stream, nullptr, nullptr)) != hipSuccess)
      return hip_fail(e, "shared gate launch");
  }
  // the kernel forms of moe_experts_forward (a caller's routing: up to N k
  // routes per expert), so that one rank's partial and this give its bits
  if ((rc = run_experts(cfg, n_rows, x, nullptr, has_sh ? shared : nullptr, nullptr, nullptr, out,
                        ws, L, stream, nullptr, n_rows * cfg->top_k, RUN_COMBINE, partial_sum)))
    return rc;
  return ok();
}

int moe_layer_forward(const moe_cfg *cfg, int32_t n_rows, const void *x, const void *router_w,
                      const float *corr_bias, const moe_expert_tables *experts,
                      const moe_shared_expert *shared, void *out, float *logits,
                      int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                      hipStream_t stream, hipEvent_t *ev) {
  return moe_layer_forward_norm(cfg, n_rows, x, nullptr, nullptr, 0.f, router_w, corr_bias,
                                experts, shared, out, logits, topk_idx, topk_w, ws, ws_bytes,
                                stream, ev);
}

int moe_layer_forward_norm(const moe_cfg *cfg, int32_t n_rows, const void *x,
                           const void *router_norm_w, const void *expert_norm_w, float eps,
                           const void *router_w, const float *corr_bias,
                           const moe_expert_tables *experts, const moe_shared_expert *shared,
                           void *out, float *logits, int32_t *topk_idx, float *topk_w, void *ws,
                           size_t ws_bytes, hipStream_t stream, hipEvent_t *ev) {
  int rc;
  Layout L;
  if ((rc = check_cfg(cfg, n_rows)) || (rc = check_ws(cfg, n_rows, ws, ws_bytes, &L)))
    return rc;
  float *lg = logits ? logits : at<float>(ws, L.logits);
  int32_t *idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float *w = topk_w ? topk_w : at<float>(ws, L.w);
  if ((rc = check_route_args(cfg, x, router_w, corr_bias, lg, idx, w)) ||
      (rc = check_expert_args(cfg, x, experts, shared, out)))
    return rc;
  const bool normed = router_norm_w || expert_norm_w;
  if (normed && !(eps >= 0.f && eps <= 1.f))
    return fail(MOE_EINVAL_SHAPE, "eps must be in [0, 1]");
  if ((router_norm_w && !aligned(router_norm_w, 16)) || (expert_norm_w && !aligned(expert_norm_w, 16)))
    return fail(MOE_EINVAL_ALIGN, "norm weights must be 16-byte aligned");
  hipError_t e;
  const void *xr = x, *xe = x;
  const bool fused = normed && router_norms_fused(n_rows, cfg->hidden, cfg->act_dtype == MOE_DT_F32);
  if (normed && !fused) {
    NormArgs na{};
    na.x = x;
    na.wr = router_norm_w;
    na.we = expert_norm_w;
    na.xr = at<void>(ws, L.xr);
    na.xe = at<void>(ws, L.xe);
    na.N = n_rows;
    na.h = cfg->hidden;
    na.eps = eps;
    if ((e = launch_rmsnorm(cfg->act_dtype == MOE_DT_F32, na, stream, evi(ev, 0), nullptr)) !=
        hipSuccess)
      return hip_fail(e, "norm launch");
    if (router_norm_w) xr = na.xr;
    if (expert_norm_w) xe = na.xe;
  }
  RouteLaunch r = route_launch(cfg, n_rows, xr, router_w, corr_bias, lg, idx, w, ws, L, shared);
  r.gx = x;  // the shared-expert gate reads the layer's own input
  r.do_router = 1;
  r.do_topk = 1;
  r.do_compact = 1;
  if (fused) {  // the router computes both norms and writes the experts' rows
    r.wr = router_norm_w;
    r.we = expert_norm_w;
    r.xe = at<void>(ws, L.xe);
    r.eps = eps;
    if (expert_norm_w) xe = r.xe;
  }
  if ((e = launch_route(r, stream, normed && !fused ? nullptr : evi(ev, 0), evi(ev, 1))) !=
      hipSuccess)
    return hip_fail(e, "routing launch");
  // top-k picks distinct experts per row: at most N routes per expert
  if ((rc = run_experts(cfg, n_rows, xe, experts, shared, idx, w, out, ws, L, stream, ev, n_rows)))
    return rc;
  return ok();
}

int moe_layer_forward_static(const moe_cfg *cfg, int32_t n_rows, const void *x,
                             const void *router_w, const float *corr_bias,
                             const moe_expert_tables *experts, const moe_shared_expert *shared,
                             void *out, float *logits, int32_t *topk_idx, float *topk_w,
                             hipStream_t stream, hipEvent_t *ev) {
  int rc;
  if ((rc = check_cfg(cfg, n_rows))) return rc;
  const Layout L = layout(*cfg, n_rows);
  if (L.total > MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE,
                "this configuration at n_rows=%d needs %zu bytes of workspace; the static "
                "scratch holds %zu",
                n_rows, L.total, (size_t)MOE_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  int dev = -1;
  if ((rc = static_scratch(&ws, &dev))) return rc;
  // the argument checks of moe_layer_forward, before anything is enqueued
  float *lg = logits ? logits : at<float>(ws, L.logits);
  int32_t *idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float *w = topk_w ? topk_w : at<float>(ws, L.w);
  if ((rc = check_route_args(cfg, x, router_w, corr_bias, lg, idx, w)) ||
      (rc = check_expert_args(cfg, x, experts, shared, out)))
    return rc;
  if ((rc = clear_static_counters(ws, dev, stream))) return rc;
  return moe_layer_forward(cfg, n_rows, x, router_w, corr_bias, experts, shared, out, logits,
                           topk_idx, topk_w, ws, MOE_STATIC_SCRATCH_BYTES, stream, ev);
}

int moe_layer_forward_hash(const moe_cfg *cfg, int32_t n_rows, const void *x,
                           const int32_t *token_ids, const int32_t *tid2eid, int32_t vocab,
                           const void *router_w, const moe_expert_tables *experts,
                           const moe_shared_expert *shared, void *out, float *logits,
                           int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t *ev) {
  int rc;
  Layout L;
  if ((rc = check_cfg(cfg, n_rows)) || (rc = check_ws(cfg, n_rows, ws, ws_bytes, &L)))
    return rc;
  float *lg = logits ? logits : at<float>(ws, L.logits);
  int32_t *idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float *w = topk_w ? topk_w : at<float>(ws, L.w);
  if ((rc = check_route_args(cfg, x, router_w, nullptr, lg, idx, w)) ||
      (rc = check_expert_args(cfg, x, experts, shared, out)))
    return rc;
  if (cfg->zero_experts) return fail(MOE_EINVAL_SHAPE, "hash routing takes no zero experts");
  if (!token_ids || !tid2eid) return fail(MOE_EINVAL_NULL, "token_ids / tid2eid is NULL");
  if (!aligned(token_ids, 4) || !aligned(tid2eid, 4))
    return fail(MOE_EINVAL_ALIGN, "token_ids and tid2eid must be 4-byte aligned");
  if (vocab < 1) return fail(MOE_EINVAL_SHAPE, "vocab must be >= 1");
  hipError_t e;
  RouteLaunch r = route_launch(cfg, n_rows, x, router_w, nullptr, lg, idx, w, ws, L, shared);
  r.token_ids = token_ids;
  r.tid2eid = tid2eid;
  r.vocab = vocab;
  r.do_router = 1;
  r.do_topk = 1;
  r.do_compact = 1;
  if ((e = launch_route(r, stream, evi(ev, 0), evi(ev, 1))) != hipSuccess)
    return hip_fail(e, "routing launch");
  // a table row may repeat an expert
  if ((rc = run_experts(cfg, n_rows, x, experts, shared, idx, w, out, ws, L, stream, ev,
                        n_rows * cfg->top_k)))
    return rc;
  return ok();
}

const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL_NULL: return "a required pointer is NULL";
    case MOE_EINVAL_SHAPE: return "a size is out of range";
    case MOE_EINVAL_TOPK: return "top_k out of range";
    case MOE_EINVAL_DTYPE: return "unsupported dtype or scoring";
    case MOE_EINVAL_ALIGN: return "misaligned pointer";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return MOE_ABI_VERSION; }

}  // extern "C"
