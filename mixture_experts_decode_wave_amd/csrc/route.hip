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
constexpr int TT = 128;       // token tile of the compaction walk
constexpr int TTW = TT / 32;  // bitmap words per expert
constexpr int ROUTER_THREADS = 256;
constexpr int EB = 4;         // experts per router workgroup
constexpr int TB = 16;        // token rows per pass

__device__ __forceinline__ uint32_t orderable(float f) {
  f = f + 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, WAVE);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, WAVE);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

template <int PER>
__device__ void topk_row(const float *__restrict__ lg, const float *__restrict__ bias, int E,
                         int k, int scoring, int norm, float rsf, int32_t *__restrict__ idx_row,
                         float *__restrict__ w_row, int lane) {
  float lv[PER];
  uint32_t key[PER];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + WAVE * i;
    lv[i] = 0.f;
    key[i] = 0;
    if (e < E) {
      lv[i] = lg[e];
      const float kf = scoring == 1 ? sigmoidf_(lv[i]) + (bias ? bias[e] : 0.f) : lv[i];
      key[i] = orderable(kf);
      avail |= 1u << i;
    }
  }
  int my_e = -1;  // lane j keeps the expert of slot j
  float my_l = 0.f;
  for (int j = 0; j < k; j++) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      if (avail & (1u << i)) {
        const uint64_t p = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)(lane + WAVE * i));
        best = p > best ? p : best;
      }
    }
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    if ((e % WAVE) == lane) avail &= ~(1u << (e / WAVE));
    if (lane == j) my_e = e;
  }
  if (lane < k) my_l = lg[my_e];
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
    const float s = lane < k ? sigmoidf_(my_l) : 0.f;
    v = norm ? s / wave_sum(s) : s;
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
};

// Top-k (optional), shared gate values (optional) and compaction, by one
// workgroup of NT threads.
template <int NT>
__device__ void topk_and_compact(const RouteArgs &a) {
  constexpr int NW = NT / WAVE;
  __shared__ int cnt[MAXE];
  __shared__ uint32_t bm[MAXE * TTW];
  __shared__ int wave_tot[NW];
  const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
  const int N = a.N, E = a.E, k = a.k, NK = a.N * a.k;

  if (a.do_topk) {
    for (int t = wave; t < N; t += NW)
      topk_any(a.logits + (size_t)t * E, a.bias, E, k, a.scoring, a.norm, a.rsf,
               a.idx + (size_t)t * k, a.w + (size_t)t * k, lane);
  }
  if (a.gate_vec) {
    for (int t = wave; t < N; t += NW) {
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
  __syncthreads();  // idx written above is read below by other waves
  if (!a.do_compact) return;

  for (int e = tid; e < MAXE; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < NK; r += NT) {
    const int e = a.idx[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // experts e = tid + NT * q
  constexpr int EPT = MAXE / NT;
  int my_cnt[EPT], base[EPT], slot[EPT];
  int n_active = 0, n_routes = 0;
#pragma unroll
  for (int q = 0; q < EPT; q++) {
    const int e = tid + NT * q;
    my_cnt[q] = e < E ? cnt[e] : 0;
    int ta, tr;
    slot[q] = block_exclusive_scan<NT>(my_cnt[q] > 0 ? 1 : 0, wave_tot, &ta) + n_active;
    base[q] = block_exclusive_scan<NT>(my_cnt[q], wave_tot, &tr) + n_routes;
    n_active += ta;
    n_routes += tr;
    if (my_cnt[q] > 0) {
      a.c.active[slot[q]] = e;
      a.c.off[slot[q]] = base[q];
    }
  }
  if (tid == 0) {
    *a.c.n_active = n_active;
    a.c.off[n_active] = n_routes;
  }

  for (int t0 = 0; t0 < N; t0 += TT) {
    const int nt = min(TT, N - t0);
    for (int i = tid; i < E * TTW; i += NT) bm[i] = 0;
    __syncthreads();
    for (int r = tid; r < nt * k; r += NT) {
      const int tl = r / k;
      const int e = a.idx[(size_t)t0 * k + r];
      if (e >= 0 && e < E)
        atomicOr(&bm[e * TTW + tl / 32], 1u << (tl % 32));
      else
        a.c.route_pos[(size_t)t0 * k + r] = -1;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < EPT; q++) {
      const int e = tid + NT * q;
      if (my_cnt[q] > 0) {
        for (int wd = 0; wd < TTW; wd++) {
          uint32_t bits = bm[e * TTW + wd];
          while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1;
            const int t = t0 + wd * 32 + b;
            for (int j = 0; j < k; j++) {
              const int src = t * k + j;
              if (a.idx[src] == e) {
                a.c.route_tok[base[q]] = t;
                a.c.route_src[base[q]] = src;
                a.c.route_pos[src] = base[q];
                base[q]++;
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }
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
  const bool fuse = r.do_router && r.N <= FUSE_MAX_N;
  if (r.do_router) {
    a.do_topk = fuse ? r.do_topk : 0;
    a.do_compact = fuse ? r.do_compact : 0;
    if (!fuse) a.gate_vec = nullptr;
    const int C = r.act_f32 ? r.h / 4 : r.h / 8;
    const int cpl = ((C + 3) / 4 + WAVE - 1) / WAVE;  // chunks per lane
    dim3 grid((r.E + EB - 1) / EB), block(ROUTER_THREADS);
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
  }
  if (!r.do_topk && !r.do_compact) return hipSuccess;
  a.do_topk = r.do_topk;
  a.do_compact = r.do_compact;
  a.gate_vec = r.gate_vec;
  hipExtLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, r.do_router ? nullptr : ev0, ev1,
                        0, a);
  return hipGetLastError();
}

}  // namespace moe
