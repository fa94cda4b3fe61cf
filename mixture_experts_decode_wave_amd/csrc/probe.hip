// Streaming-read probe: the rate at which this GPU reads a large buffer with
// plain 128-bit loads and does nothing else.  It is the practical ceiling the
// expert passes' weight streams are measured beside (the published 8 TB/s is
// their peak); it computes nothing of the layer.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "../../include/moe_wave.h"
#include "device.h"

namespace moe {
namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_U = 8;  // 16-byte loads in flight per thread

// Workgroup b reads 16-byte chunks b*256 + tid + i*stride (grid-stride, 8 loads
// issued per trip before any is used).  The XOR of everything a thread read
// is stored only if it equals a value no buffer of this probe produces (the
// caller's buffer is zero-filled), so the loads cannot be dropped and the
// probe writes next to nothing.
__global__ __launch_bounds__(PROBE_THREADS) void stream_read_kernel(const u32x4 *buf,
                                                                    size_t chunks,
                                                                    uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  for (; i + (PROBE_U - 1) * stride < chunks; i += PROBE_U * stride) {
    u32x4 v[PROBE_U];
#pragma unroll
    for (int u = 0; u < PROBE_U; u++) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < PROBE_U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < chunks; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * PROBE_THREADS + threadIdx.x] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t grid,
                                     hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (!buf || !sink) return MOE_EINVAL_NULL;
  if ((uintptr_t)buf % 16 || bytes % 16 || (uintptr_t)sink % 4) return MOE_EINVAL_ALIGN;
  if (grid < 1 || grid > 65536) return MOE_EINVAL_SHAPE;
  hipExtLaunchKernelGGL(moe::stream_read_kernel, dim3(grid), dim3(moe::PROBE_THREADS), 0, stream,
                        ev0, ev1, 0, (const moe::u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
