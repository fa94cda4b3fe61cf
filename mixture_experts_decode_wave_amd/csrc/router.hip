// Router GEMV: logits[t, e] = sum_i x[t, i] * W[e, i] for every token row t.
//
// The router step of MoeLayer::forward (forward.rs, decode_gate_gemv) and of
// grouped_route (forward_fp8_grouped_router.rs).  That page's per-row router
// re-read the whole router once per group of <= 16 rows; here one wave owns
// one expert row of W for ALL N token rows, so W crosses HBM exactly once
// per launch whatever N is.  The token rows are the reused operand: they
// stay hot in L2 and are streamed per wave in groups of TG rows.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int ROUTER_THREADS = 256;
constexpr int ROUTER_WAVES = ROUTER_THREADS / WAVE;
constexpr int TG = 8;  // token rows accumulated together

template <bool F32>
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

template <bool F32>
__global__ __launch_bounds__(ROUTER_THREADS) void router_gemv_kernel(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ W, float *__restrict__ logits, int N,
    int E, int C /* 16-byte chunks per row */) {
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int e = blockIdx.x * ROUTER_WAVES + wave;
  if (e >= E) return;  // the whole wave leaves; no block barrier below
  const u32x4 *wrow = W + (size_t)e * C;
  for (int t0 = 0; t0 < N; t0 += TG) {
    float acc[TG];
#pragma unroll
    for (int i = 0; i < TG; i++) acc[i] = 0.f;
    const int nt = min(TG, N - t0);
    for (int c = lane; c < C; c += WAVE) {
      const u32x4 wv = __builtin_nontemporal_load(wrow + c);
#pragma unroll
      for (int i = 0; i < TG; i++)
        if (i < nt) acc[i] = chunk_dot<F32>(wv, x[(size_t)(t0 + i) * C + c], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < TG; i++) {
      if (i < nt) {
        const float s = wave_sum(acc[i]);
        if (lane == 0) logits[(size_t)(t0 + i) * E + e] = s;
      }
    }
  }
}

}  // namespace

hipError_t launch_router(bool act_f32, const void *x, const void *W, float *logits, int N, int E,
                         int h, hipStream_t s) {
  const int C = act_f32 ? h / 4 : h / 8;
  dim3 grid((E + ROUTER_WAVES - 1) / ROUTER_WAVES), block(ROUTER_THREADS);
  if (act_f32)
    hipLaunchKernelGGL(router_gemv_kernel<true>, grid, block, 0, s, (const u32x4 *)x,
                       (const u32x4 *)W, logits, N, E, C);
  else
    hipLaunchKernelGGL(router_gemv_kernel<false>, grid, block, 0, s, (const u32x4 *)x,
                       (const u32x4 *)W, logits, N, E, C);
  return hipGetLastError();
}

}  // namespace moe
