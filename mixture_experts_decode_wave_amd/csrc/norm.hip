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

// 16-byte chunks per thread: h <= 16384 is 2048 bf16 chunks or 4096 fp32 ones
template <bool F32>
constexpr int kNormCpt = F32 ? 16 : 8;

// fp32 values of a 16-byte chunk: 8 bf16 or 4 fp32 (then v[4..7] unused)
template <bool F32>
__device__ __forceinline__ void unpack(const u32x4 &c, float (&v)[8]) {
  if constexpr (F32) {
    v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
  } else {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; q++) { v[2 * q] = bf16_lo(w[q]); v[2 * q + 1] = bf16_hi(w[q]); }
  }
}

template <bool F32>
__device__ __forceinline__ u32x4 pack(const float (&v)[8]) {
  if constexpr (F32)
    return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                 __float_as_uint(v[3])};
  else
    return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
}

// The row's chunks are all loaded at once (with the weights'), so a row costs
// one memory round trip before its sum of squares, which is summed per
// thread, per wave, then over the waves in a fixed order.
template <bool F32>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_kernel(NormArgs a) {
  constexpr int EPC = F32 ? 4 : 8;  // elements per chunk
  __shared__ float part[NORM_THREADS / WAVE];
  const int t = blockIdx.x;
  const int C = a.h / EPC;  // h % 32 == 0
  const u32x4 *X = (const u32x4 *)a.x + (size_t)t * C;
  constexpr int NORM_CPT = kNormCpt<F32>;
  u32x4 xc[NORM_CPT], rc[NORM_CPT], ec[NORM_CPT];
#pragma unroll
  for (int u = 0; u < NORM_CPT; u++) {
    const int c = min((int)threadIdx.x + u * NORM_THREADS, C - 1);
    xc[u] = X[c];
    rc[u] = a.wr ? ((const u32x4 *)a.wr)[c] : u32x4{0, 0, 0, 0};
    ec[u] = a.we ? ((const u32x4 *)a.we)[c] : u32x4{0, 0, 0, 0};
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NORM_CPT; u++) {
    float v[8];
    unpack<F32>(xc[u], v);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; e++) q = fmaf(v[e], v[e], q);
    ss += (int)threadIdx.x + u * NORM_THREADS < C ? q : 0.f;
  }
  ss = wave_sum(ss);
  if (threadIdx.x % WAVE == 0) part[threadIdx.x / WAVE] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NORM_THREADS / WAVE; w++) tot += part[w];
  const float r = 1.0f / sqrtf(tot / (float)a.h + a.eps);
#pragma unroll
  for (int u = 0; u < NORM_CPT; u++) {
    const int c = (int)threadIdx.x + u * NORM_THREADS;
    if (c >= C) break;
    float v[8], wv[8], o[8];
    unpack<F32>(xc[u], v);
    if (a.wr) {
      unpack<F32>(rc[u], wv);
#pragma unroll
      for (int e = 0; e < EPC; e++) o[e] = v[e] * r * wv[e];
      ((u32x4 *)a.xr)[(size_t)t * C + c] = pack<F32>(o);
    }
    if (a.we) {
      unpack<F32>(ec[u], wv);
#pragma unroll
      for (int e = 0; e < EPC; e++) o[e] = v[e] * r * wv[e];
      ((u32x4 *)a.xe)[(size_t)t * C + c] = pack<F32>(o);
    }
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
