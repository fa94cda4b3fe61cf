// The layer's optional pre-norms (forward.rs: the router reads its input
// through a pre-norm when the layer has one, and the pre_expert_norm step
// normalises the experts' input after routing; the shared-expert gate keeps
// the layer's own input).  RMSNorm:
//   y[t, i] = x[t, i] * w[i] / sqrt(mean_i x[t, i]^2 + eps)
// computed in fp32 and stored in the activation dtype, as a separate norm
// step would hand it on.  One workgroup per row; both weight vectors in one
// pass over the row.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int NORM_THREADS = 256;

template <bool F32>
__device__ __forceinline__ float load_act(const void *p, size_t i) {
  if constexpr (F32) return ((const float *)p)[i];
  else return bf16_lo(((const uint16_t *)p)[i]);
}

template <bool F32>
__device__ __forceinline__ void store_act(void *p, size_t i, float v) {
  if constexpr (F32) ((float *)p)[i] = v;
  else ((uint16_t *)p)[i] = (uint16_t)f32_to_bf16_bits(v);
}

template <bool F32>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_kernel(NormArgs a) {
  __shared__ float part[NORM_THREADS / WAVE];
  const int t = blockIdx.x;
  const size_t row = (size_t)t * a.h;
  // sum of squares: each thread a strided slice, then the wave, then the waves
  // in a fixed order
  float ss = 0.f;
  for (int i = threadIdx.x; i < a.h; i += NORM_THREADS) {
    const float v = load_act<F32>(a.x, row + i);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (threadIdx.x % WAVE == 0) part[threadIdx.x / WAVE] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NORM_THREADS / WAVE; w++) tot += part[w];
  const float r = 1.0f / sqrtf(tot / (float)a.h + a.eps);
  for (int i = threadIdx.x; i < a.h; i += NORM_THREADS) {
    const float v = load_act<F32>(a.x, row + i) * r;
    if (a.wr) store_act<F32>(a.xr, row + i, v * load_act<F32>(a.wr, i));
    if (a.we) store_act<F32>(a.xe, row + i, v * load_act<F32>(a.we, i));
  }
}

}  // namespace

hipError_t launch_rmsnorm(bool act_f32, const NormArgs &a, hipStream_t s, hipEvent_t e0,
                          hipEvent_t e1) {
  if (act_f32)
    hipExtLaunchKernelGGL(rmsnorm_kernel<true>, dim3(a.N), dim3(NORM_THREADS), 0, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL(rmsnorm_kernel<false>, dim3(a.N), dim3(NORM_THREADS), 0, s, e0, e1, 0,
                          a);
  return hipGetLastError();
}

}  // namespace moe
