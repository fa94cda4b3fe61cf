// Top-k selection and route compaction, one 1024-thread workgroup.
//
// Top-k follows the scoring the pages' batched kernels take
// (forward_token_major.rs: moe_topk_softmax_batched with norm_topk_prob,
// moe_topk_sigmoid_batched with a correction bias, norm_topk_prob and
// routed_scaling_factor): one wave per logits row; every lane holds up to 16
// experts' keys as order-preserving u32 codes packed with the complemented
// expert id into a 64-bit word, so a wave-wide max picks the largest key and,
// among equal keys, the lowest expert id.  k rounds give the slots in
// descending key order.
//
// Compaction groups the N*k (token, slot) routes by expert -- experts in
// ascending id, routes of one expert in ascending (token, slot) -- so the
// expert kernels stream each selected expert's weights once for all of its
// routes (the pages' token-major decode instead walks every route and reads
// an expert once per route).  Counting is a histogram in LDS; positions come
// from a per-expert walk over a token bitmap, which makes the order, and so
// every later sum, independent of thread timing.
#include <limits.h>

#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int RT_THREADS = 1024;
constexpr int RT_WAVES = RT_THREADS / WAVE;
constexpr int MAXE = 1024;
constexpr int PER_LANE = MAXE / WAVE;  // keys per lane
constexpr int TT = 128;                // token tile of the compaction walk
constexpr int TTW = TT / 32;           // bitmap words per expert

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

__device__ void topk_row(const float *__restrict__ lg, const float *__restrict__ bias, int E,
                         int k, int scoring, int norm, float rsf, int32_t *__restrict__ idx_row,
                         float *__restrict__ w_row, int lane) {
  float lv[PER_LANE];
  uint32_t key[PER_LANE];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; i++) {
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
  for (int j = 0; j < k; j++) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; i++) {
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
  // weights of the k picks (lanes 0..k-1)
  const float l = lane < k ? lg[my_e] : 0.f;
  float v;
  if (scoring == 0) {
    const float m = __shfl(l, 0, WAVE);  // slot 0 holds the largest logit
    const float p = lane < k ? expf(l - m) : 0.f;
    float den;
    if (norm) {
      den = wave_sum(p);
    } else {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < PER_LANE; i++)
        if (lane + WAVE * i < E) z += expf(lv[i] - m);
      den = wave_sum(z);
    }
    v = p / den;
  } else {
    const float s = lane < k ? sigmoidf_(l) : 0.f;
    v = norm ? s / wave_sum(s) : s;
  }
  if (lane < k) {
    idx_row[lane] = my_e;
    w_row[lane] = v * rsf;
  }
}

// exclusive prefix sum over the block of one int per thread; returns the
// block total through *total
__device__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
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
  for (int w = 0; w < RT_WAVES; w++) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

struct RouteArgs {
  const float *logits;
  const float *bias;
  int32_t *idx;
  float *w;
  int N, E, k, scoring, norm;
  float rsf;
  int do_topk, do_compact;
  Compact c;
};

__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  __shared__ int cnt[MAXE];
  __shared__ uint32_t bm[MAXE * TTW];
  __shared__ int wave_tot[RT_WAVES];
  const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
  const int N = a.N, E = a.E, k = a.k, NK = a.N * a.k;

  if (a.do_topk) {
    for (int t = wave; t < N; t += RT_WAVES)
      topk_row(a.logits + (size_t)t * E, a.bias, E, k, a.scoring, a.norm, a.rsf,
               a.idx + (size_t)t * k, a.w + (size_t)t * k, lane);
    __syncthreads();  // idx written above is read below by other waves
  }
  if (!a.do_compact) return;

  for (int e = tid; e < MAXE; e += RT_THREADS) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < NK; r += RT_THREADS) {
    const int e = a.idx[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // one expert per thread (E <= 1024 = RT_THREADS)
  const int my_cnt = tid < E ? cnt[tid] : 0;
  int n_active, n_routes;
  const int slot = block_exclusive_scan(my_cnt > 0 ? 1 : 0, wave_tot, &n_active);
  int base = block_exclusive_scan(my_cnt, wave_tot, &n_routes);
  if (my_cnt > 0) {
    a.c.active[slot] = tid;
    a.c.off[slot] = base;
  }
  if (tid == 0) {
    *a.c.n_active = n_active;
    a.c.off[n_active] = n_routes;
  }

  for (int t0 = 0; t0 < N; t0 += TT) {
    const int nt = min(TT, N - t0);
    for (int i = tid; i < E * TTW; i += RT_THREADS) bm[i] = 0;
    __syncthreads();
    for (int r = tid; r < nt * k; r += RT_THREADS) {
      const int tl = r / k;
      const int e = a.idx[(size_t)t0 * k + r];
      if (e >= 0 && e < E)
        atomicOr(&bm[e * TTW + tl / 32], 1u << (tl % 32));
      else
        a.c.route_pos[(size_t)t0 * k + r] = -1;
    }
    __syncthreads();
    if (my_cnt > 0) {
      for (int wd = 0; wd < TTW; wd++) {
        uint32_t bits = bm[tid * TTW + wd];
        while (bits) {
          const int b = __builtin_ctz(bits);
          bits &= bits - 1;
          const int t = t0 + wd * 32 + b;
          for (int j = 0; j < k; j++) {
            const int src = t * k + j;
            if (a.idx[src] == tid) {
              a.c.route_tok[base] = t;
              a.c.route_src[base] = src;
              a.c.route_pos[src] = base;
              base++;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route(const float *logits, const float *bias, int32_t *idx, float *w, int N,
                        int E, int k, int scoring, int norm, float rsf, bool do_topk,
                        bool do_compact, const Compact &c, hipStream_t s) {
  RouteArgs a{logits, bias, idx, w, N, E, k, scoring, norm, rsf, do_topk ? 1 : 0,
              do_compact ? 1 : 0, c};
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(RT_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
