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
// experts' keys as order-preserving u32 codes.  A bit-by-bit ballot search
// finds a threshold that at least k lane maxima reach; the keys at or above
// it (usually about k) are gathered in LDS in ascending expert id, and each
// ranks itself by the candidates that beat it (a larger key, or an equal key
// at a lower id).  Ranks below k are the picks and a pick's rank is its
// slot, so equal keys go to the lowest id and slots run in descending key
// order.
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

// LDS a wave's top-k uses to gather candidates and to put its k picks in
// slot order.
struct __attribute__((aligned(16))) TopkScratch {
  uint32_t key[WAVE];  // read in blocks of 8: n <= 64 stays within the arrays
  int id[WAVE];
  float logit[WAVE];
  int slot_id[WAVE];
  float slot_logit[WAVE];
};

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// How many of the n (key, id) pairs in LDS beat (key, id): a larger key, or
// an equal key at a lower id.  Broadcast reads, 8 pairs per loop trip (a
// rolled loop keeps this once-per-launch code small; the reads of a trip are
// issued together).
__device__ __forceinline__ int beaten_by(const TopkScratch &ts, int n, uint32_t key, int id) {
  int r = 0;
#pragma unroll 1
  for (int q = 0; q < n; q += 8) {
    const u32x4 k0 = *(const u32x4 *)&ts.key[q];
    const u32x4 k1 = *(const u32x4 *)&ts.key[q + 4];
    const u32x4 i0 = *(const u32x4 *)&ts.id[q];
    const u32x4 i1 = *(const u32x4 *)&ts.id[q + 4];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const uint32_t ku = u < 4 ? k0[u & 3] : k1[u & 3];
      const int iu = (int)(u < 4 ? i0[u & 3] : i1[u & 3]);
      r += (q + u < n) && (ku > key || (ku == key && iu < id));
    }
  }
  return r;
}

// A threshold T with at least k of the wave's values v >= T: the largest
// such T, or one with exactly k values >= T (the search stops there: the set
// {v >= T} no longer changes).  Bit by bit from the top, by ballot counts.
__device__ __forceinline__ uint32_t kth_threshold(uint32_t v, int k) {
  uint32_t T = 0;
  for (int b = 31; b >= 0; b--) {
    const uint32_t c = T | (1u << b);
    const int cnt = __popcll(__ballot(v >= c));
    if (cnt >= k) {
      T = c;
      if (cnt == k) break;
    }
  }
  return T;
}

// One logits row by one wave.  Lane l holds experts l + 64 i (i < PER) as
// order-preserving u32 keys (0 = not available).
//  1. T1, a threshold with at least k lane maxima >= T1 (bit by bit, ballot
//     counts), bounds the k-th largest key from below, so every pick is among
//     the keys >= T1: usually about k of them.
//  2. The candidates are gathered one per lane in LDS; a candidate's rank is
//     the number of candidates that beat it (larger key, or equal key at a
//     lower expert id).  The picks are the ranks below k, and a pick's slot is
//     its rank: descending key order, equal keys in ascending id.
// With more than 64 candidates (heavy ties) the picks come from a bitwise
// search for the k-th largest key over all keys instead.
template <int PER>
__device__ void topk_row(const float *__restrict__ lg, const float *__restrict__ bias, int E,
                         int k, int scoring, int norm, float rsf, int32_t *__restrict__ idx_row,
                         float *__restrict__ w_row, int lane, TopkScratch &ts, int *idx_lds) {
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
  // 1. T1
  uint32_t lm = key[0];
#pragma unroll
  for (int i = 1; i < PER; i++) lm = max(lm, key[i]);
  // at least k lane maxima are >= T1, so the k-th largest key is too
  const uint32_t T1 = kth_threshold(lm, k);
  int n_cand = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) n_cand += __popcll(__ballot(key[i] >= T1));

  int slot = WAVE;  // this lane's pick's slot (WAVE: no pick), its id and logit
  int cid = 0;
  float cl = 0.f;
  if (n_cand <= WAVE) {
    // 2. candidates, in ascending expert id
    int before = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const bool c = key[i] >= T1;
      const uint64_t m = __ballot(c);
      if (c) {
        const int pos = before + lanes_below(m);
        ts.key[pos] = key[i];
        ts.id[pos] = lane + WAVE * i;
        ts.logit[pos] = lv[i];
      }
      before += __popcll(m);
    }
    wave_lds_sync();
    if (lane < n_cand) {
      cid = ts.id[lane];
      cl = ts.logit[lane];
      const int r = beaten_by(ts, n_cand, ts.key[lane], cid);
      if (r < k) slot = r;
    }
  } else {
    // 2'. the k-th largest key T bit by bit; the keys > T and the lowest-id
    // keys == T are the picks, gathered at lanes 0..k-1 and ranked there
    uint32_t T = 0;
    for (int b = 31; b >= 0; b--) {
      const uint32_t c = T | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PER; i++) cnt += __popcll(__ballot(key[i] >= c));
      if (cnt >= k) T = c;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) n_gt += __popcll(__ballot(key[i] > T));
    const int need = k - n_gt;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const uint64_t eqm = __ballot(key[i] == T);
      const bool sel = key[i] > T || (key[i] == T && eq_before + lanes_below(eqm) < need);
      const uint64_t selm = __ballot(sel);
      if (sel) {
        const int pos = sel_before + lanes_below(selm);
        ts.key[pos] = key[i];
        ts.id[pos] = lane + WAVE * i;
        ts.logit[pos] = lv[i];
      }
      eq_before += __popcll(eqm);
      sel_before += __popcll(selm);
    }
    wave_lds_sync();
    if (lane < k) {
      cid = ts.id[lane];
      cl = ts.logit[lane];
      slot = beaten_by(ts, k, ts.key[lane], cid);
    }
  }
  if (slot < WAVE) {
    ts.slot_id[slot] = cid;
    ts.slot_logit[slot] = cl;
  }
  wave_lds_sync();
  const int my_e = lane < k ? ts.slot_id[lane] : 0;
  const float my_l = lane < k ? ts.slot_logit[lane] : 0.f;
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
    if (idx_lds) idx_lds[lane] = my_e;
  }
}

__device__ void topk_any(const float *lg, const float *bias, int E, int k, int scoring, int norm,
                         float rsf, int32_t *idx_row, float *w_row, int lane, TopkScratch &ts,
                         int *idx_lds) {
  if (E <= 2 * WAVE)
    topk_row<2>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane, ts, idx_lds);
  else if (E <= 4 * WAVE)
    topk_row<4>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane, ts, idx_lds);
  else if (E <= 8 * WAVE)
    topk_row<8>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane, ts, idx_lds);
  else
    topk_row<16>(lg, bias, E, k, scoring, norm, rsf, idx_row, w_row, lane, ts, idx_lds);
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
  int N, E, h, act_f32;  // E: router width (real experts, then zero experts)
  int Er;                // real experts: ids [Er, E) are zero experts, never routes
  const float *bias;
  int32_t *idx;
  float *w;
  int k, scoring, norm;
  float rsf;
  int do_topk, do_compact;
  Compact c;
  uint32_t *counter;     // zeroed workspace word; back to 0 after every launch
  const void *gate_vec;  // shared-expert gate vector [h] (act dtype) or NULL
  const void *gx;        // [N, h] rows the gate vector reads
  const int32_t *token_ids;  // hash routing: [N] token ids, or NULL (top-k)
  const int32_t *tid2eid;    // hash routing: [vocab, k] expert table
  int vocab;
  float *g;              // g[t] = sigmoid(gx_t . gate_vec)
  float *part;           // [S][N][E] partial logits of the K-split router, or NULL
  int S;                 // K slices of part
  // pre-norms computed inside the VALU router (router_kernel<..., true>):
  // RMSNorm weights of the router's input and of the experts' (nullable), the
  // experts' normed rows [N, h] written here, and epsilon
  const void *wr, *we;
  void *xe;
  float eps;
};

// logits row t: the logits buffer, or the sum of the router's K-slice
// partials in slice order (written back to the logits buffer)
__device__ __forceinline__ const float *logits_row(const RouteArgs &a, int t, int lane) {
  float *row = a.logits + (size_t)t * a.E;
  if (a.part) {
    // 4 experts x 8 slices per lane per trip, every load of a trip issued
    // before the sums: one memory round trip per trip (E = 512 and 8 slices:
    // two trips, not eight)
#pragma unroll 1
    for (int e0 = lane; e0 < a.E; e0 += 4 * WAVE) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int s0 = 0; s0 < a.S; s0 += 8) {
        float p[4][8];
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const int e = min(e0 + q * WAVE, a.E - 1), sl = min(s0 + u, a.S - 1);
            p[q][u] = a.part[((size_t)sl * a.N + t) * a.E + e];
          }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int u = 0; u < 8; u++)
            if (s0 + u < a.S) v[q] += p[q][u];  // slice order
      }
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (e0 + q * WAVE < a.E) row[e0 + q * WAVE] = v[q];
    }
  }
  return row;
}

// Hash routing of row t by one wave (forward.rs, the hash-routing branch of
// the top-k step): the experts are row token_ids[t] of tid2eid, each weighted
// by sqrt(softplus(logit)) at it, renormalised if norm, times rsf.  An entry
// outside [0, E) is dropped (weight 0; the compaction skips it); a token id
// outside [0, vocab) drops its whole row (ids -1).
__device__ void hash_row(const RouteArgs &a, const float *row, int t, int lane, int *idx_lds) {
  const int tok = a.token_ids[t];
  const bool tok_ok = tok >= 0 && tok < a.vocab;
  int e = -1;
  float sc = 0.f;
  if (lane < a.k && tok_ok) {
    e = a.tid2eid[(size_t)tok * a.k + lane];
    if (e >= 0 && e < a.E) {
      const float z = row[e];
      sc = sqrtf(z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z)));
    }
  }
  float v = sc;
  if (a.norm) {
    const float sum = wave_sum(sc);
    v = sum > 0.f ? sc / sum : 0.f;
  }
  if (lane < a.k) {
    a.idx[(size_t)t * a.k + lane] = e;
    a.w[(size_t)t * a.k + lane] = v * a.rsf;
    if (idx_lds) idx_lds[t * a.k + lane] = e;
  }
}

// Top-k of rows t = t0, t0 + step, ... (one wave per row) and the shared
// expert's gate values of those rows.  idx_lds (nullable, N*k <= 64 entries)
// receives a copy of the picks for a compaction in the same workgroup.
__device__ void topk_rows(const RouteArgs &a, int t0, int step, TopkScratch &ts, int *idx_lds) {
  const int lane = threadIdx.x % WAVE;
  for (int t = t0; t < a.N; t += step) {
    if (a.do_topk && a.token_ids) {
      const float *row = logits_row(a, t, lane);
      // lanes read logits other lanes of this wave may just have written
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      hash_row(a, row, t, lane, idx_lds);
    } else if (a.do_topk) {
      const float *row = logits_row(a, t, lane);
      topk_any(row, a.bias, a.E, a.k, a.scoring, a.norm, a.rsf, a.idx + (size_t)t * a.k,
               a.w + (size_t)t * a.k, lane, ts, idx_lds ? idx_lds + t * a.k : nullptr);
    }
    if (a.gate_vec) {
      // 16-byte chunks, 4 per lane per trip with every load of a trip issued
      // before the sums (a row of h <= 16384 takes at most 8 trips)
      const int C = a.act_f32 ? a.h / 4 : a.h / 8;
      const u32x4 *X = (const u32x4 *)a.gx + (size_t)t * C;
      const u32x4 *G = (const u32x4 *)a.gate_vec;
      float d = 0.f;
#pragma unroll 1
      for (int c0 = lane; c0 < C; c0 += 4 * WAVE) {
        u32x4 xa[4], ga[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int c = min(c0 + u * WAVE, C - 1);
          xa[u] = X[c];
          ga[u] = G[c];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          float q = 0.f;
          if (a.act_f32) {
            q = fmaf(__uint_as_float(xa[u].x), __uint_as_float(ga[u].x), q);
            q = fmaf(__uint_as_float(xa[u].y), __uint_as_float(ga[u].y), q);
            q = fmaf(__uint_as_float(xa[u].z), __uint_as_float(ga[u].z), q);
            q = fmaf(__uint_as_float(xa[u].w), __uint_as_float(ga[u].w), q);
          } else {
            q = dot2(xa[u].x, ga[u].x, q);
            q = dot2(xa[u].y, ga[u].y, q);
            q = dot2(xa[u].z, ga[u].z, q);
            q = dot2(xa[u].w, ga[u].w, q);
          }
          d += c0 + u * WAVE < C ? q : 0.f;
        }
      }
      d = wave_sum(d);
      if (lane == 0) a.g[t] = sigmoidf_(d);
    }
  }
}

// Route compaction of at most 64 routes by wave 0 alone (a pick outside the
// Er real experts -- a zero expert, or a dropped id -- is no route): lane r
// holds route r = t k + j with key (expert << 16 | r); its position is the number
// of smaller keys, an expert's slot the number of experts with a smaller id.
// The keys go through LDS and every lane reads them all (broadcast reads, in
// rolled loops: this code runs once per launch, with a cold instruction cache).
// idx_lds: the picks of this workgroup's top-k (else they are read from a.idx).
__device__ void compact_small(const RouteArgs &a, const int *idx_lds) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[WAVE];
  if (threadIdx.x >= WAVE) return;
  const int lane = threadIdx.x;
  const int NK = a.N * a.k;
  const int e = lane < NK ? (idx_lds ? idx_lds[lane] : a.idx[lane]) : -1;
  const bool valid = lane < NK && e >= 0 && e < a.Er;
  const uint32_t key = valid ? ((uint32_t)e << 16) | (uint32_t)lane : 0xFFFFFFFFu;
  keys[lane] = key;
  wave_lds_sync();
  int rank = 0, lower_same = 0;
#pragma unroll 1
  for (int q = 0; q < NK; q += 8) {  // keys past NK are all-ones: never smaller
    const u32x4 k0 = *(const u32x4 *)&keys[q];
    const u32x4 k1 = *(const u32x4 *)&keys[q + 4];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const uint32_t kr = u < 4 ? k0[u & 3] : k1[u & 3];
      rank += kr < key;
      lower_same += kr < key && (kr >> 16) == (key >> 16);
    }
  }
  const bool first = valid && lower_same == 0;
  const uint64_t fmask = __ballot(first);
  int slot = 0;
#pragma unroll 1
  for (int q = 0; q < NK; q += 8) {
    const u32x4 k0 = *(const u32x4 *)&keys[q];
    const u32x4 k1 = *(const u32x4 *)&keys[q + 4];
    const uint32_t fb = (uint32_t)(fmask >> q);
#pragma unroll
    for (int u = 0; u < 8; u++)
      slot += ((fb >> u) & 1) && ((u < 4 ? k0[u & 3] : k1[u & 3]) >> 16) < (key >> 16);
  }
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
__device__ void compact(const RouteArgs &a, const int *idx_lds) {
  constexpr int NW = NT / WAVE;
  constexpr int RT = 256;        // routes per tile
  constexpr int RW = RT / 32;    // bitmap words per expert
  __shared__ int cnt[MAXE];      // routes per expert, then running base
  __shared__ uint32_t bm[MAXE * RW];
  __shared__ int wave_tot[NW];
  const int tid = threadIdx.x;
  const int E = a.Er, NK = a.N * a.k;  // real experts: zero-expert picks are not routes
  if (NK <= WAVE) {
    compact_small(a, idx_lds);
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

// Multi-workgroup compaction (steps of more than PAR_COMPACT_MIN_GROUPS
// groups of 16 rows), in three steps that give every route the position the
// one-workgroup compaction gives it: (expert ascending, then token, then
// slot).
//
// 1. Top-k workgroup g (rows [16 g, 16 g + 16)) counts its routes per expert:
//    hist[e][g].
__device__ void route_histogram(const RouteArgs &a) {
  __shared__ int cnt[MAXE];
  const int g = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int r0 = 16 * g * a.k, r1 = min(16 * g + 16, a.N) * a.k;
  for (int e = tid; e < a.Er; e += nt) cnt[e] = 0;
  __syncthreads();  // also: this workgroup's picks, written above, are visible
  for (int r = r0 + tid; r < r1; r += nt) {
    const int e = a.idx[r];
    if (e >= 0 && e < a.Er) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int GS = hist_stride(a.N);
  for (int e = tid; e < a.Er; e += nt) a.c.hist[(size_t)e * GS + g] = cnt[e];
}

// 2. The last workgroup to arrive: per expert, the exclusive prefix over the
//    groups plus the expert's first position replaces hist[e][g]; the active
//    experts, their first positions and counts as the one-workgroup
//    compaction writes them.  One thread per expert, 16-byte loads, 16 in
//    flight.
template <int NT>
__device__ void hist_scan(const RouteArgs &a) {
  __shared__ int wave_tot[NT / WAVE];
  const int tid = threadIdx.x, G = (a.N + 15) / 16, GS = hist_stride(a.N);
  constexpr int EPT = MAXE / NT;
  int tot[EPT];
#pragma unroll
  for (int q = 0; q < EPT; q++) {
    const int e = tid + NT * q;
    int t = 0;
    if (e < a.Er) {
      const int4 *row = (const int4 *)(a.c.hist + (size_t)e * GS);
      for (int c0 = 0; c0 < GS / 4; c0 += 16) {
        int4 v[16];
#pragma unroll
        for (int u = 0; u < 16; u++) v[u] = row[min(c0 + u, GS / 4 - 1)];
#pragma unroll
        for (int u = 0; u < 16; u++) {
          const int g = 4 * (c0 + u);
          if (c0 + u < GS / 4) {
            t += (g < G ? v[u].x : 0) + (g + 1 < G ? v[u].y : 0) + (g + 2 < G ? v[u].z : 0) +
                 (g + 3 < G ? v[u].w : 0);
          }
        }
      }
    }
    tot[q] = t;
  }
  int n_active = 0, n_routes = 0, base[EPT];
#pragma unroll
  for (int q = 0; q < EPT; q++) {
    const int e = tid + NT * q;
    int ta, tr;
    const int slot = block_exclusive_scan<NT>(tot[q] > 0 ? 1 : 0, wave_tot, &ta) + n_active;
    base[q] = block_exclusive_scan<NT>(tot[q], wave_tot, &tr) + n_routes;
    n_active += ta;
    n_routes += tr;
    if (tot[q] > 0) {
      a.c.active[slot] = e;
      a.c.off[slot] = base[q];
    }
  }
  if (tid == 0) {
    *a.c.n_active = n_active;
    a.c.off[n_active] = n_routes;
  }
#pragma unroll
  for (int q = 0; q < EPT; q++) {
    const int e = tid + NT * q;
    if (e >= a.Er || tot[q] == 0) continue;
    int4 *row = (int4 *)(a.c.hist + (size_t)e * GS);
    int run = base[q];
    for (int c0 = 0; c0 < GS / 4; c0 += 16) {
      int4 v[16];
#pragma unroll
      for (int u = 0; u < 16; u++) v[u] = row[min(c0 + u, GS / 4 - 1)];
#pragma unroll
      for (int u = 0; u < 16; u++) {
        const int g = 4 * (c0 + u);
        if (c0 + u < GS / 4) {
          int4 o;
          o.x = run; run += g < G ? v[u].x : 0;
          o.y = run; run += g + 1 < G ? v[u].y : 0;
          o.z = run; run += g + 2 < G ? v[u].z : 0;
          o.w = run; run += g + 3 < G ? v[u].w : 0;
          row[c0 + u] = o;
        }
      }
    }
  }
}

// 3. Workgroup g places its routes: a route's position is hist[e][g] plus the
//    number of the group's earlier routes (t k + j order) of the same expert.
constexpr int SCATTER_THREADS = 512;  // 16 rows x k <= 32 routes

__global__ __launch_bounds__(SCATTER_THREADS) void scatter_kernel(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) int el[SCATTER_THREADS];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int r0 = 16 * g * a.k, nr = (min(16 * g + 16, a.N) - 16 * g) * a.k;
  const int e = tid < nr ? a.idx[r0 + tid] : -1;
  const bool valid = e >= 0 && e < a.Er;
  el[tid] = valid ? e : -1;
  __syncthreads();
  if (tid >= nr) return;
  if (!valid) {
    a.c.route_pos[r0 + tid] = -1;
    return;
  }
  int rank = 0;
#pragma unroll 1
  for (int i = 0; i < nr; i += 4) {  // broadcast reads; entries past nr are -1
    const int4 v = *(const int4 *)&el[i];
    rank += (i < tid && v.x == e) + (i + 1 < tid && v.y == e) + (i + 2 < tid && v.z == e) +
            (i + 3 < tid && v.w == e);
  }
  const int p = a.c.hist[(size_t)e * hist_stride(a.N) + g] + rank;
  a.c.route_tok[p] = (r0 + tid) / a.k;
  a.c.route_src[p] = r0 + tid;
  a.c.route_pos[r0 + tid] = p;
}

// Top-k of all rows, gate values and compaction, by one workgroup.
template <int NT>
__device__ void topk_and_compact(const RouteArgs &a) {
  __shared__ TopkScratch ts[NT / WAVE];
  __shared__ int idx_lds[WAVE];
  const bool small = a.do_topk && a.N * a.k <= WAVE;
  topk_rows(a, threadIdx.x / WAVE, NT / WAVE, ts[threadIdx.x / WAVE], small ? idx_lds : nullptr);
  __syncthreads();  // idx written above is read below by other waves
  if (!a.do_compact) return;
  if (a.N == 1 && a.do_topk && !a.token_ids && a.Er == a.E) {
    // one row under top-k routing without zero experts: its k routes are k
    // distinct experts, so route position = slot.  Each expert's weights still cross HBM once,
    // and every item's results stand alone, so the experts' order changes
    // no result; the ranking is skipped.
    const int j = threadIdx.x;
    if (j < a.k) {
      a.c.active[j] = idx_lds[j];
      a.c.off[j] = j;
      a.c.route_tok[j] = 0;
      a.c.route_src[j] = j;
      a.c.route_pos[j] = j;
    }
    if (j == 0) {
      *a.c.n_active = a.k;
      a.c.off[a.k] = a.k;
    }
    return;
  }
  compact<NT>(a, small ? idx_lds : nullptr);
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

// fp32 values of a 16-byte chunk (8 bf16, or 4 fp32: then v[4..7] unset)
template <bool F32>
__device__ __forceinline__ void chunk_vals(const u32x4 &c, float (&v)[8]) {
  if constexpr (F32) {
    v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
  } else {
    v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x); v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
    v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z); v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
  }
}

// The chunk x * r * w, stored in the activation dtype (RMSNorm's output)
template <bool F32>
__device__ __forceinline__ u32x4 chunk_norm(const u32x4 &x, const u32x4 &w, float r) {
  float v[8], g[8];
  chunk_vals<F32>(x, v);
  chunk_vals<F32>(w, g);
  if constexpr (F32)
    return u32x4{__float_as_uint(v[0] * r * g[0]), __float_as_uint(v[1] * r * g[1]),
                 __float_as_uint(v[2] * r * g[2]), __float_as_uint(v[3] * r * g[3])};
  else
    return u32x4{pack_bf16x2(v[0] * r * g[0], v[1] * r * g[1]),
                 pack_bf16x2(v[2] * r * g[2], v[3] * r * g[3]),
                 pack_bf16x2(v[4] * r * g[4], v[5] * r * g[5]),
                 pack_bf16x2(v[6] * r * g[6], v[7] * r * g[7])};
}

template <bool F32>
__device__ __forceinline__ float chunk_sumsq(const u32x4 &x) {
  float v[8];
  chunk_vals<F32>(x, v);
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < (F32 ? 4 : 8); e++) q = fmaf(v[e], v[e], q);
  return q;
}

// Workgroup b: experts [b*EB, b*EB + EB); wave w: chunks of quarter w of the
// row; lane: chunks c = qbeg + lane + 64 i (i < CPL).
//
// NORM: the layer's pre-norms as well (forward.rs, MoeLayer::forward: the
// router's input through its pre-norm, and the pre_expert_norm step).  A
// workgroup holds whole rows, so it forms each row's sum of squares itself
// (lane, then 16-lane row, then the 16 row sums in order), the router reads the rows
// normed with the router's weights, and workgroup b writes its share of the
// experts' normed rows (chunks [b CPW, b CPW + CPW)) for the expert passes.
// NORM takes N <= 4 (one group of rows).
template <bool F32, int CPL, bool NORM>
__global__ __launch_bounds__(ROUTER_THREADS) void router_kernel(RouteArgs a) {
  __shared__ float part[ROUTER_THREADS / 16][EB][TB];
  __shared__ float ssq[NORM ? ROUTER_THREADS / 16 : 1][4];
  __shared__ int last;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int C = F32 ? a.h / 4 : a.h / 8;  // 16-byte chunks per row
  const int CQ = (C + 3) / 4;             // chunks per quarter
  const int qbeg = wave * CQ, qend = min(C, qbeg + CQ);
  const int e0 = blockIdx.x * EB;
  const u32x4 *W = (const u32x4 *)a.W;
  const u32x4 *X = (const u32x4 *)a.x;

  // Every load below is unconditional, from a clamped in-bounds address, and
  // no loaded value is tested before the sums, so the compiler issues the W
  // and x loads back to back and waits once.  A chunk past the quarter (C is
  // a multiple of 4, so no quarter is empty) is left out of the sums; an
  // expert past E or a row past N repeats the last one and is not stored.
  u32x4 wv[EB][CPL];
  bool on[CPL];
#pragma unroll
  for (int i = 0; i < CPL; i++) on[i] = qbeg + lane + WAVE * i < qend;
  // NORM (N <= 4): the rows and the norm weights are loaded before W, so the
  // norms are formed while the W loads are in flight.  These loads are
  // unconditional, from clamped addresses (a missing weight vector reads x
  // instead, unused), so nothing delays the W loads behind them.
  const int cpw = (C + gridDim.x - 1) / gridDim.x;  // experts' chunks per workgroup
  const int cb = blockIdx.x * cpw;
  u32x4 xn[NORM ? 4 : 1][NORM ? CPL : 1], gr[NORM ? CPL : 1];
  u32x4 xx[NORM ? 4 : 1], xg;  // thread j: chunk cb + j of the experts' rows
  if constexpr (NORM) {
    const u32x4 *WR = (const u32x4 *)(a.wr ? a.wr : a.x);
    const u32x4 *WE = (const u32x4 *)(a.we ? a.we : a.x);
#pragma unroll
    for (int i = 0; i < CPL; i++) {
      const int c = min(qbeg + lane + WAVE * i, qend - 1);
#pragma unroll
      for (int t = 0; t < 4; t++) xn[t][i] = X[(size_t)min(t, a.N - 1) * C + c];
      gr[i] = WR[c];
    }
    const int c = min(cb + (int)threadIdx.x, C - 1);
#pragma unroll
    for (int t = 0; t < 4; t++) xx[t] = X[(size_t)min(t, a.N - 1) * C + c];
    xg = WE[c];
  }
#pragma unroll
  for (int eb = 0; eb < EB; eb++)
#pragma unroll
    for (int i = 0; i < CPL; i++)
      wv[eb][i] = __builtin_nontemporal_load(W + (size_t)min(e0 + eb, a.E - 1) * C +
                                             min(qbeg + lane + WAVE * i, qend - 1));
  if constexpr (NORM) {
    float rs[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; i++) q += on[i] ? chunk_sumsq<F32>(xn[t][i]) : 0.f;
      q = group_sum<16>(q);  // DPP only; the 16 row sums meet in LDS
      if ((lane & 15) == 0) ssq[wave * 4 + lane / 16][t] = q;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; t++) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < ROUTER_THREADS / 16; w++) tot += ssq[w][t];
      rs[t] = 1.0f / sqrtf(tot / (float)a.h + a.eps);
    }
    if (a.we) {  // the workgroup's chunks [cb, cb + cpw) of the experts' rows
      for (int j = threadIdx.x; j < cpw; j += ROUTER_THREADS) {
        const int c = cb + j;
        if (c >= C) break;
        const bool first = j == (int)threadIdx.x;
        const u32x4 gv = first ? xg : ((const u32x4 *)a.we)[c];
#pragma unroll
        for (int t = 0; t < 4; t++)
          if (t < a.N)
            ((u32x4 *)a.xe)[(size_t)t * C + c] =
                chunk_norm<F32>(first ? xx[t] : X[(size_t)t * C + c], gv, rs[t]);
      }
    }
    if (a.wr) {
#pragma unroll
      for (int t = 0; t < 4; t++)
#pragma unroll
        for (int i = 0; i < CPL; i++) xn[t][i] = chunk_norm<F32>(xn[t][i], gr[i], rs[t]);
    }
  }
  for (int t0 = 0; t0 < a.N; t0 += TB) {
    const int nt = min(TB, a.N - t0);
    float acc[EB][TB];
#pragma unroll
    for (int eb = 0; eb < EB; eb++)
#pragma unroll
      for (int t = 0; t < TB; t++) acc[eb][t] = 0.f;
#pragma unroll
    for (int tq = 0; tq < TB; tq += 4) {  // rows in groups of 4: one round trip each
      if (tq < nt) {
        u32x4 xv[4][CPL];
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
          for (int i = 0; i < CPL; i++) {
            if constexpr (NORM)
              xv[t][i] = xn[t][i];
            else
              xv[t][i] = X[(size_t)(t0 + min(tq + t, nt - 1)) * C + min(qbeg + lane + WAVE * i, qend - 1)];
          }
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
          for (int i = 0; i < CPL; i++)
#pragma unroll
            for (int eb = 0; eb < EB; eb++) {
              const float d = chunk_dot<F32, CPL>(wv[eb][i], xv[t][i], acc[eb][tq + t]);
              acc[eb][tq + t] = on[i] ? d : acc[eb][tq + t];
            }
      }
    }
    // sums within each 16-lane row (DPP only), then the 16 row sums of a
    // logit (4 waves x 4 rows) in a fixed order through LDS
#pragma unroll
    for (int t = 0; t < TB; t++) {
      if (t < nt) {
#pragma unroll
        for (int eb = 0; eb < EB; eb++) {
          const float s = group_sum<16>(acc[eb][t]);
          if ((lane & 15) == 0) part[wave * 4 + lane / 16][eb][t] = s;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < EB * TB) {
      const int eb = threadIdx.x / TB, t = threadIdx.x % TB;
      if (t < nt && e0 + eb < a.E) {
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r++) v += part[r][eb][t];
        a.logits[(size_t)(t0 + t) * a.E + e0 + eb] = v;
      }
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

// Top-k of 16 rows per workgroup (one row per wave), then the compaction:
// PAR, steps 1 and 2 of the multi-workgroup form (scatter_kernel follows);
// else all of it in the last workgroup to arrive.
template <bool PAR>
__global__ __launch_bounds__(1024) void topk_kernel(RouteArgs a) {
  __shared__ int last;
  __shared__ TopkScratch ts[16];
  topk_rows(a, blockIdx.x * 16 + threadIdx.x / WAVE, a.N, ts[threadIdx.x / WAVE],
            nullptr);  // one row per wave
  if (!a.do_compact) return;
  if constexpr (PAR) route_histogram(a);
  if (!arrive_last(a.counter, gridDim.x, true, &last)) return;
  if constexpr (PAR)
    hist_scan<1024>(a);
  else
    compact<1024>(a, nullptr);
}

// The top-k launch (16 rows a workgroup) and, for large steps, the scatter
// of the multi-workgroup compaction.  ev0 / ev1 as for launch_route.
hipError_t launch_topk(const RouteArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = (a.N + 15) / 16;
  const bool par = a.do_compact && G > PAR_COMPACT_MIN_GROUPS;
  if (!par) {
    hipExtLaunchKernelGGL(topk_kernel<false>, dim3(G), dim3(1024), 0, s, ev0, ev1, 0, a);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(topk_kernel<true>, dim3(G), dim3(1024), 0, s, ev0, nullptr, 0, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(scatter_kernel, dim3(G), dim3(SCATTER_THREADS), 0, s, nullptr, ev1, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteLaunch &r, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  RouteArgs a{};
  a.x = r.x;
  a.W = r.W;
  a.logits = r.logits;
  a.N = r.N;
  a.E = r.E;
  a.Er = r.Er;
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
  a.gx = r.gx ? r.gx : r.x;
  a.token_ids = r.token_ids;
  a.tid2eid = r.tid2eid;
  a.vocab = r.vocab;
  a.g = r.g;
  a.do_topk = r.do_topk;
  a.do_compact = r.do_compact;
  if (!r.do_router) {  // top-k and / or compaction of given logits / indices
    if (!r.do_topk && !r.do_compact && !r.gate_vec) return hipSuccess;
    if (r.N > FUSE_MAX_N) return launch_topk(a, s, ev0, ev1);
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
    const bool norm = r.wr || r.we;
    if (norm) {  // router_norms_fused() holds: cpl <= 4
      a.wr = r.wr;
      a.we = r.we;
      a.xe = r.xe;
      a.eps = r.eps;
    }
#define MOE_ROUTER(F, P, NM) \
  hipExtLaunchKernelGGL((router_kernel<F, P, NM>), grid, block, 0, s, ev0, stop, 0, a)
    if (norm) {
      if (r.act_f32) {
        if (cpl <= 1) MOE_ROUTER(true, 1, true);
        else if (cpl <= 2) MOE_ROUTER(true, 2, true);
        else MOE_ROUTER(true, 4, true);
      } else {
        if (cpl <= 1) MOE_ROUTER(false, 1, true);
        else if (cpl <= 2) MOE_ROUTER(false, 2, true);
        else MOE_ROUTER(false, 4, true);
      }
    } else if (r.act_f32) {
      if (cpl <= 1) MOE_ROUTER(true, 1, false);
      else if (cpl <= 2) MOE_ROUTER(true, 2, false);
      else if (cpl <= 4) MOE_ROUTER(true, 4, false);
      else MOE_ROUTER(true, 8, false);
    } else {
      if (cpl <= 1) MOE_ROUTER(false, 1, false);
      else if (cpl <= 2) MOE_ROUTER(false, 2, false);
      else if (cpl <= 4) MOE_ROUTER(false, 4, false);
      else MOE_ROUTER(false, 8, false);
    }
#undef MOE_ROUTER
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse) return e;
    a.do_topk = r.do_topk;
    a.do_compact = r.do_compact;
    a.gate_vec = r.gate_vec;
    return launch_topk(a, s, nullptr, ev1);
  }
  // K-split MFMA router, then top-k over N/16 workgroups
  const int KS = router_kslice(r.h, r.E);
  a.S = (r.h + KS - 1) / KS;
  a.part = r.part;
  hipExtLaunchKernelGGL(router_mfma_kernel, dim3((r.E + 15) / 16, a.S), dim3(256), 0, s, ev0,
                        nullptr, 0, a, KS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk(a, s, nullptr, ev1);
}

// The router computes the pre-norms itself for N <= FUSE_MAX_N rows of up to
// 4 chunks per lane (h <= 8192 in bf16, 4096 in fp32); larger steps and
// longer rows take them from the norm kernel.
bool router_norms_fused(int N, int h, bool act_f32) {
  if (N > FUSE_MAX_N) return false;
  const int C = act_f32 ? h / 4 : h / 8;
  return ((C + 3) / 4 + WAVE - 1) / WAVE <= 4;
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
