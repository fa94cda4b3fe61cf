// Router GEMV, top-k selection and route compaction.
//
// Router: logits[t, e] = sum_i x[t, i] * W[e, i] (MoeLayer::forward's
// decode_gate_gemv; grouped_route in forward_fp8_grouped_router.rs).  That
// page's per-row router re-read the whole router once per group of <= 16
// rows; here a workgroup owns EB expert rows for ALL N token rows, so W
// crosses HBM exactly once per launch whatever N is.  The 4 waves of a
// workgroup split the hidden dimension in quarters (their partial sums meet
// in LDS); each lane keeps its W chunks in registers and streams the token
// rows, which stay hot in L2.
//
// Top-k follows the scoring of the pages' batched kernels
// (forward_token_major.rs: moe_topk_softmax_batched with norm_topk_prob,
// moe_topk_sigmoid_batched with a correction bias, norm_topk_prob and
// routed_scaling_factor): one wave per logits row; every lane holds up to 16
// experts' keys as order-preserving u32 codes packed with the complemented
// expert id into a 64-bit word, so a wave-wide max picks the largest key and,
// among equal keys, the lowest expert id; k rounds give the slots in
// descending key order.
//
// Compaction groups the N*k (token, slot) routes by expert -- experts in
// ascending id, routes of one expert in ascending (token, slot) -- so the
// expert kernels stream each selected expert's weights once for all of its
// routes (the token-major decode on the pages walks every route and reads an
// expert once per route).  Counting is an LDS histogram; positions come from
// a per-expert walk over a token bitmap, so the order, and every later sum,
// does not depend on thread timing.
//
// For N <= FUSE_MAX_N the workgroup that finishes the router last (a
// self-resetting counter in the workspace) goes on with top-k and
// compaction, which saves a launch; otherwise a 1024-thread kernel does them.
#include <limits.h>

#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int MAXE = 1024;
constexpr int ROUTER_THREADS = 256;
constexpr int EB = 4;         // experts per router workgroup
constexpr int TB = 16;        // token rows per pass

__device__ __forceinline__ uint32_t orderable(float f) {
  f = f + 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest u32 of the wave, in every lane (DPP within rows, row broadcasts
// toward lane 63, readlane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_QUAD_1032>(v));
  v = max(v, dpp_u32<DPP_QUAD_2301>(v));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));
  v = max(v, dpp_u32<DPP_ROW_BCAST15, 0xA>(v));
  v = max(v, dpp_u32<DPP_ROW_BCAST31, 0xC>(v));
  return __builtin_amdgcn_readlane(v, WAVE - 1);
}

// One logits row by one wave.  Lane l holds experts l + 64 i (i < PER) as
// order-preserving u32 keys (0 = not available).  A round takes the wave-wide
// largest key, then the lowest expert id holding it (ballots over i, lowest
// lane), and retires it; k rounds give the slots in descending key order with
// equal keys in ascending id.
template <int PER>
__device__ void topk_row(const float *__restrict__ lg, const float *__restrict__ bias, int E,
                         int k, int scoring, int norm, float rsf, int32_t *__restrict__ idx_row,
                         float *__restrict__ w_row, int lane) {
  float lv[PER];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + WAVE * i;
    lv[i] = e < E ? lg[e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + WAVE * i;
    key[i] = 0;
    if (e < E) {
      const float kf = scoring == 1 ? sigmoidf_(lv[i]) + (bias ? bias[e] : 0.f) : lv[i];
      key[i] = orderable(kf);
    }
  }
  int my_e = 0;  // lane j keeps the expert of slot j
  for (int j = 0; j < k; j++) {
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < PER; i++) lm = max(lm, key[i]);
    const uint32_t wm = wave_max_u32(lm);
    int e = -1;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const uint64_t m = __ballot(key[i] == wm);
      if (e < 0 && m) e = WAVE * i + __builtin_ctzll(m);
    }
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (e == lane + WAVE * i) key[i] = 0;
    if (lane == j) my_e = e;
  }
  // logits of the k picks, from the lanes that hold them
  float my_l = 0.f;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const float v = __shfl(lv[i], my_e % WAVE, WAVE);
    if (my_e / WAVE == i) my_l = v;
  }
  float v;
  if (scoring == 0) {
    const float m = __shfl(my_l, 0, WAVE);  // slot 0 holds the largest logit
    const float p = lane < k ? expf(my_l - m) : 0.f;
    float den;
    if (norm) {
      den = wave_sum(p);
    } else {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < PER; i++)
        if (lane + WAVE * i < E) z += expf(lv[i] - m);
      den = wave_sum(z);
    }
    v = p / den;
  } else {
    const float sg = lane < k ? sigmoidf_(my_l) : 0.f;
    v = norm ? sg / wave_sum(sg) : sg;
  }
  if (lane < k) {
    idx_row[lane] = my_e;
    w_row[lane] = v * rsf;
  }
}

__device__ void topk_any(const float *lg, const float *bias, int E, int k, int scoring, int norm,
                         float rsf, int32_t *idx_row, float *w_row, int lane) {
  if (E <= 2 * WAVE)
    topk_row<2>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane);
  else if (E <= 4 * WAVE)
    topk_row<4>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane);
  else if (E <= 8 * WAVE)
    topk_row<8>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane);
  else
    topk_row<16>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane);
}

// exclusive prefix sum over the block of one int per thread (values for
// threads >= nthreads count as given); returns the block total via *total
template <int NT>
__device__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
  int inc = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int u = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += u;
  }
  if (lane == WAVE - 1) wave_tot[wave] = inc;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < NW; w++) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

struct RouteArgs {
  const void *x;
  const void *W;
  float *logits;
  int N, E, h, act_f32;
  const float *bias;
  int32_t *idx;
  float *w;
  int k, scoring, norm;
  float rsf;
  int do_topk, do_compact;
  Compact c;
  uint32_t *counter;     // zeroed workspace word; back to 0 after every launch
  const void *gate_vec;  // shared-expert gate vector [h] (act dtype) or NULL
  float *g;              // g[t] = sigmoid(x_t . gate_vec)
  float *part;           // [S][N][E] partial logits of the K-split router, or NULL
  int S;                 // K slices of part
};

// logits row t: the logits buffer, or the sum of the router's K-slice
// partials in slice order (written back to the logits buffer)
__device__ __forceinline__ const float *logits_row(const RouteArgs &a, int t, int lane) {
  float *row = a.logits + (size_t)t * a.E;
  if (a.part) {
    for (int e = lane; e < a.E; e += WAVE) {
      float v = 0.f;
      for (int s0 = 0; s0 < a.S; s0 += 8) {
        float p[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
          p[u] = s0 + u < a.S ? a.part[((size_t)(s0 + u) * a.N + t) * a.E + e] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; u++) v += p[u];  // slice order; + 0 beyond S is exact
      }
      row[e] = v;
    }
  }
  return row;
}

// Top-k of rows t = t0, t0 + step, ... (one wave per row) and the shared
// expert's gate values of those rows.
__device__ void topk_rows(const RouteArgs &a, int t0, int step) {
  const int lane = threadIdx.x % WAVE;
  for (int t = t0; t < a.N; t += step) {
    if (a.do_topk) {
      const float *row = logits_row(a, t, lane);
      topk_any(row, a.bias, a.E, a.k, a.scoring, a.norm, a.rsf, a.idx + (size_t)t * a.k,
               a.w + (size_t)t * a.k, lane);
    }
    if (a.gate_vec) {
      float d = 0.f;
      for (int i = lane; i < a.h; i += WAVE) {
        float xv, gv;
        if (a.act_f32) {
          xv = ((const float *)a.x)[(size_t)t * a.h + i];
          gv = ((const float *)a.gate_vec)[i];
        } else {
          xv = bf16_lo(((const uint16_t *)a.x)[(size_t)t * a.h + i]);
          gv = bf16_lo(((const uint16_t *)a.gate_vec)[i]);
        }
        d = fmaf(xv, gv, d);
      }
      d = wave_sum(d);
      if (lane == 0) a.g[t] = sigmoidf_(d);
    }
  }
}

// Route compaction of at most 64 routes by wave 0 alone: lane r holds
// route r = t k + j, its position is its rank by (expert, r), an expert's
// slot the number of experts with a smaller id.  No barriers, no LDS.
__device__ void compact_small(const RouteArgs &a) {
  if (threadIdx.x >= WAVE) return;
  const int lane = threadIdx.x;
  const int NK = a.N * a.k;
  const int e = lane < NK ? a.idx[lane] : -1;
  const bool valid = lane < NK && e >= 0 && e < a.E;
  const uint32_t key = valid ? ((uint32_t)e << 16) | (uint32_t)lane : 0xFFFFFFFFu;
  int rank = 0, lower_same = 0;
  for (int r = 0; r < NK; r++) {
    const uint32_t kr = __builtin_amdgcn_readlane(key, r);
    rank += kr < key;
    lower_same += kr < key && (kr >> 16) == (key >> 16);
  }
  const bool first = valid && lower_same == 0;
  const uint64_t fmask = __ballot(first);
  int slot = 0;
  for (int r = 0; r < NK; r++)
    if ((fmask >> r) & 1) slot += (__builtin_amdgcn_readlane(key, r) >> 16) < (key >> 16);
  const int n_valid = __popcll(__ballot(valid));
  const int n_active = __popcll(fmask);
  if (valid) {
    a.c.route_tok[rank] = lane / a.k;
    a.c.route_src[rank] = lane;
    a.c.route_pos[lane] = rank;
  } else if (lane < NK) {
    a.c.route_pos[lane] = -1;
  }
  if (first) {
    a.c.active[slot] = e;
    a.c.off[slot] = rank;
  }
  if (lane == 0) {
    *a.c.n_active = n_active;
    a.c.off[n_active] = n_valid;
  }
}

// Route compaction by one workgroup of NT threads (idx of every row written
// and visible to it): an LDS histogram and scans give each expert's first
// position; then, tile by tile of RT routes, a per-expert bitmap over the
// tile's routes gives every route its rank among its expert's routes.
template <int NT>
__device__ void compact(const RouteArgs &a) {
  constexpr int NW = NT / WAVE;
  constexpr int RT = 256;        // routes per tile
  constexpr int RW = RT / 32;    // bitmap words per expert
  __shared__ int cnt[MAXE];      // routes per expert, then running base
  __shared__ uint32_t bm[MAXE * RW];
  __shared__ int wave_tot[NW];
  const int tid = threadIdx.x;
  const int E = a.E, NK = a.N * a.k;
  if (NK <= WAVE) {
    compact_small(a);
    return;
  }

  for (int e = tid; e < MAXE; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < NK; r += NT) {
    const int e = a.idx[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // experts e = tid + NT * q: slots and first positions
  constexpr int EPT = MAXE / NT;
  int my_cnt[EPT], base[EPT];
  int n_active = 0, n_routes = 0;
#pragma unroll
  for (int q = 0; q < EPT; q++) {
    const int e = tid + NT * q;
    my_cnt[q] = e < E ? cnt[e] : 0;
    int ta, tr;
    const int slot = block_exclusive_scan<NT>(my_cnt[q] > 0 ? 1 : 0, wave_tot, &ta) + n_active;
    base[q] = block_exclusive_scan<NT>(my_cnt[q], wave_tot, &tr) + n_routes;
    n_active += ta;
    n_routes += tr;
    if (my_cnt[q] > 0) {
      a.c.active[slot] = e;
      a.c.off[slot] = base[q];
    }
  }
  if (tid == 0) {
    *a.c.n_active = n_active;
    a.c.off[n_active] = n_routes;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < EPT; q++)
    if (tid + NT * q < MAXE) cnt[tid + NT * q] = base[q];  // first free position
  for (int r0 = 0; r0 < NK; r0 += RT) {
    for (int i = tid; i < E * RW; i += NT) bm[i] = 0;
    __syncthreads();
    for (int r = r0 + tid; r < min(NK, r0 + RT); r += NT) {
      const int e = a.idx[r];
      if (e >= 0 && e < E) atomicOr(&bm[e * RW + (r - r0) / 32], 1u << ((r - r0) % 32));
    }
    __syncthreads();
    for (int r = r0 + tid; r < min(NK, r0 + RT); r += NT) {
      const int e = a.idx[r];
      if (e >= 0 && e < E) {
        const int rl = r - r0, wd = rl / 32;
        int rank = __popc(bm[e * RW + wd] & ((1u << (rl % 32)) - 1u));
        for (int w2 = 0; w2 < wd; w2++) rank += __popc(bm[e * RW + w2]);
        const int p = cnt[e] + rank;
        a.c.route_tok[p] = r / a.k;
        a.c.route_src[p] = r;
        a.c.route_pos[r] = p;
      } else {
        a.c.route_pos[r] = -1;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
      int n = 0;
      for (int w2 = 0; w2 < RW; w2++) n += __popc(bm[e * RW + w2]);
      cnt[e] += n;
    }
    __syncthreads();
  }
}

// Top-k of all rows, gate values and compaction, by one workgroup.
template <int NT>
__device__ void topk_and_compact(const RouteArgs &a) {
  topk_rows(a, threadIdx.x / WAVE, NT / WAVE);
  __syncthreads();  // idx written above is read below by other waves
  if (a.do_compact) compact<NT>(a);
}

// ---------------------------------------------------------------- router

template <bool F32, int CPL>
__device__ __forceinline__ float chunk_dot(const u32x4 &w, const u32x4 &x, float acc) {
  if constexpr (F32) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  } else {
    acc = dot2(w.x, x.x, acc);
    acc = dot2(w.y, x.y, acc);
    acc = dot2(w.z, x.z, acc);
    acc = dot2(w.w, x.w, acc);
  }
  return acc;
}

// Workgroup b: experts [b*EB, b*EB + EB); wave w: chunks of quarter w of the
// row; lane: chunks c = qbeg + lane + 64 i (i < CPL).
template <bool F32, int CPL>
__global__ __launch_bounds__(ROUTER_THREADS) void router_kernel(RouteArgs a) {
  __shared__ float part[ROUTER_THREADS / WAVE][EB][TB];
  __shared__ int last;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int C = F32 ? a.h / 4 : a.h / 8;  // 16-byte chunks per row
  const int CQ = (C + 3) / 4;             // chunks per quarter
  const int qbeg = wave * CQ, qend = min(C, qbeg + CQ);
  const int e0 = blockIdx.x * EB;
  const u32x4 *W = (const u32x4 *)a.W;
  const u32x4 *X = (const u32x4 *)a.x;

  u32x4 wv[EB][CPL];
#pragma unroll
  for (int eb = 0; eb < EB; eb++)
#pragma unroll
    for (int i = 0; i < CPL; i++) {
      const int c = qbeg + lane + WAVE * i;
      wv[eb][i] = u32x4{0, 0, 0, 0};
      if (e0 + eb < a.E && c < qend)
        wv[eb][i] = __builtin_nontemporal_load(W + (size_t)(e0 + eb) * C + c);
    }
  for (int t0 = 0; t0 < a.N; t0 += TB) {
    const int nt = min(TB, a.N - t0);
    float acc[EB][TB];
#pragma unroll
    for (int eb = 0; eb < EB; eb++)
#pragma unroll
      for (int t = 0; t < TB; t++) acc[eb][t] = 0.f;
#pragma unroll
    for (int t = 0; t < TB; t++) {
      if (t < nt) {
#pragma unroll
        for (int i = 0; i < CPL; i++) {
          const int c = qbeg + lane + WAVE * i;
          if (c < qend) {
            const u32x4 xv = X[(size_t)(t0 + t) * C + c];
#pragma unroll
            for (int eb = 0; eb < EB; eb++) acc[eb][t] = chunk_dot<F32, CPL>(wv[eb][i], xv, acc[eb][t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TB; t++) {
      if (t < nt) {
#pragma unroll
        for (int eb = 0; eb < EB; eb++) {
          const float s = wave_sum(acc[eb][t]);
          if (lane == 0) part[wave][eb][t] = s;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < EB * TB) {
      const int eb = threadIdx.x / TB, t = threadIdx.x % TB;
      if (t < nt && e0 + eb < a.E)
        a.logits[(size_t)(t0 + t) * a.E + e0 + eb] =
            part[0][eb][t] + part[1][eb][t] + part[2][eb][t] + part[3][eb][t];
    }
    __syncthreads();
  }
  if (!a.do_topk && !a.do_compact) return;
  // the last workgroup to finish goes on with top-k and compaction
  if (!arrive_last(a.counter, gridDim.x, true, &last)) return;
  topk_and_compact<ROUTER_THREADS>(a);
}

__global__ __launch_bounds__(1024) void route_kernel(RouteArgs a) {
  topk_and_compact<1024>(a);
}

// K-split MFMA router for larger N: workgroup (eb, s) owns experts
// [16 eb, 16 eb + 16) and hidden columns [s KS, (s+1) KS) for ALL N rows, so
// every router weight is read by exactly one workgroup; its 16 x KS tile
// lives in registers as the A operand of v_mfma_f32_16x16x32_bf16 while the
// waves stream 16-row token tiles (L2-resident) as the B operand.  Partial
// logits go to part[s][t][e]; the top-k kernel sums the slices in order.
constexpr int RM_KSTEPS = 16;  // k-steps of 32 columns per slice, at most

__global__ __launch_bounds__(256) void router_mfma_kernel(RouteArgs a, int KS) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const int eb = blockIdx.x, sl = blockIdx.y;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int m16 = lane & 15, kg = lane >> 4;
  const int e = eb * 16 + m16;
  const int k0 = sl * KS;
  const int nst = (min(a.h, k0 + KS) - k0) / 32;
  const uint16_t *W = (const uint16_t *)a.W;
  const uint16_t *X = (const uint16_t *)a.x;
  u32x4 wa[RM_KSTEPS];
#pragma unroll
  for (int i = 0; i < RM_KSTEPS; i++) {
    wa[i] = u32x4{0, 0, 0, 0};
    if (i < nst && e < a.E)
      wa[i] = __builtin_nontemporal_load(
          (const u32x4 *)(W + (size_t)e * a.h + k0 + 32 * i + 8 * kg));
  }
  const int tiles = (a.N + 15) / 16;
  for (int tt = wave; tt < tiles; tt += 4) {
    const int t = tt * 16 + m16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    u32x4 xb[RM_KSTEPS];
#pragma unroll
    for (int i = 0; i < RM_KSTEPS; i++) {
      xb[i] = u32x4{0, 0, 0, 0};
      if (i < nst && t < a.N)
        xb[i] = *(const u32x4 *)(X + (size_t)t * a.h + k0 + 32 * i + 8 * kg);
    }
#pragma unroll
    for (int i = 0; i < RM_KSTEPS; i++)
      if (i < nst)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[i]),
                                                      __builtin_bit_cast(bf16x8, xb[i]), acc, 0,
                                                      0, 0);
    // lane holds experts 4 kg + j (j < 4) of the tile for token m16
    if (t < a.N) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int ej = eb * 16 + 4 * kg + j;
        if (ej < a.E) a.part[((size_t)sl * a.N + t) * a.E + ej] = acc[j];
      }
    }
  }
}

// Top-k of 16 rows per workgroup (one per wave); the last workgroup to finish
// compacts the routes of all rows.
__global__ __launch_bounds__(1024) void topk_kernel(RouteArgs a) {
  __shared__ int last;
  topk_rows(a, blockIdx.x * 16 + threadIdx.x / WAVE, a.N);  // one row per wave
  if (!a.do_compact) return;
  if (!arrive_last(a.counter, gridDim.x, true, &last)) return;
  compact<1024>(a);
}

}  // namespace

hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  RouteArgs a{};
  a.x = r.x;
  a.W = r.W;
  a.logits = r.logits;
  a.N = r.N;
  a.E = r.E;
  a.h = r.h;
  a.act_f32 = r.act_f32;
  a.bias = r.bias;
  a.idx = r.idx;
  a.w = r.w;
  a.k = r.k;
  a.scoring = r.scoring;
  a.norm = r.norm;
  a.rsf = r.rsf;
  a.c = r.c;
  a.counter = r.counter;
  a.gate_vec = r.gate_vec;
  a.g = r.g;
  a.do_topk = r.do_topk;
  a.do_compact = r.do_compact;
  if (!r.do_router) {  // top-k and / or compaction of given logits / indices
    if (!r.do_topk && !r.do_compact && !r.gate_vec) return hipSuccess;
    hipExtLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, ev0, ev1, 0, a);
    return hipGetLastError();
  }
  if (r.N <= FUSE_MAX_N || r.act_f32) {
    // VALU router; its last workgroup runs top-k and compaction
    const int C = r.act_f32 ? r.h / 4 : r.h / 8;
    const int cpl = ((C + 3) / 4 + WAVE - 1) / WAVE;  // chunks per lane
    dim3 grid((r.E + EB - 1) / EB), block(ROUTER_THREADS);
    const bool fuse = r.N <= FUSE_MAX_N;
    if (!fuse) {
      a.do_topk = 0;
      a.do_compact = 0;
      a.gate_vec = nullptr;
    }
    hipEvent_t stop = fuse ? ev1 : nullptr;
#define MOE_ROUTER(F, P) \
  hipExtLaunchKernelGGL((router_kernel<F, P>), grid, block, 0, s, ev0, stop, 0, a)
    if (r.act_f32) {
      if (cpl <= 2) MOE_ROUTER(true, 2);
      else if (cpl <= 4) MOE_ROUTER(true, 4);
      else MOE_ROUTER(true, 8);
    } else {
      if (cpl <= 2) MOE_ROUTER(false, 2);
      else if (cpl <= 4) MOE_ROUTER(false, 4);
      else MOE_ROUTER(false, 8);
    }
#undef MOE_ROUTER
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse) return e;
    a.do_topk = r.do_topk;
    a.do_compact = r.do_compact;
    a.gate_vec = r.gate_vec;
    hipExtLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, nullptr, ev1, 0, a);
    return hipGetLastError();
  }
  // K-split MFMA router, then top-k over N/16 workgroups
  const int KS = router_kslice(r.h, r.E);
  a.S = (r.h + KS - 1) / KS;
  a.part = r.part;
  hipExtLaunchKernelGGL(router_mfma_kernel, dim3((r.E + 15) / 16, a.S), dim3(256), 0, s, ev0,
                        nullptr, 0, a, KS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(topk_kernel, dim3((r.N + 15) / 16), dim3(1024), 0, s, nullptr, ev1, 0, a);
  return hipGetLastError();
}

// Hidden columns per router K slice: a multiple of 32, at most 512 (the A
// tile lives in registers), and enough slices for ~256 workgroups.
int router_kslice(int h, int E) {
  const int etiles = (E + 15) / 16;
  int S = (256 + etiles - 1) / etiles;
  const int smin = (h + 511) / 512;
  if (S < smin) S = smin;
  int KS = ((h + S - 1) / S + 31) / 32 * 32;
  if (KS > 512) KS = 512;
  if (KS < 32) KS = 32;
  return KS;
}

}  // namespace moe
