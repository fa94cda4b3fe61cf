// Device helpers shared by the gfx950 kernels of the MoE decode layer:
// vector types, bf16 packing, weight-chunk decoding (FP8 e4m3 / MXFP4 through
// the gfx950 hardware converters) and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Fmt { FMT_F32 = 0, FMT_BF16 = 1, FMT_FP8 = 2, FMT_MXFP4 = 3 };

constexpr int WAVE = 64;

// Elements of one 16-byte weight chunk.
template <int FMT>
struct ChunkElems;
template <> struct ChunkElems<FMT_F32> { static constexpr int value = 4; };
template <> struct ChunkElems<FMT_BF16> { static constexpr int value = 8; };
template <> struct ChunkElems<FMT_FP8> { static constexpr int value = 16; };
template <> struct ChunkElems<FMT_MXFP4> { static constexpr int value = 32; };

// Global-memory loads.  Casting to the global address space makes them
// global_load (not flat_load, which also counts against the LDS counter), and
// a load that falls outside its matrix reads zeros from g_zero16 instead of
// sitting in a branch: loads without control flow around them let the
// compiler wait for one k-step's data (vmcnt(N)) instead of all of it.
static __device__ __attribute__((aligned(64))) uint32_t g_zero16[16];

typedef const __attribute__((address_space(1))) u32x4 *global_u32x4_ptr;
typedef const __attribute__((address_space(1))) uint8_t *global_u8_ptr;

__device__ __forceinline__ const void *zero16() { return (const void *)g_zero16; }
__device__ __forceinline__ u32x4 gload16(const void *p) { return *(global_u32x4_ptr)p; }
__device__ __forceinline__ u32x4 gload16_nt(const void *p) {
  return __builtin_nontemporal_load((global_u32x4_ptr)p);
}
__device__ __forceinline__ uint32_t gload8(const void *p) { return *(global_u8_ptr)p; }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two of them packed (lo in bits 0-15): gfx950's v_cvt_pk_bf16_f32, which
// rounds to nearest even as f32_to_bf16_bits does.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// acc + a.lo*b.lo + a.hi*b.hi with packed bf16 operands (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), acc, false);
}

// Two OCP e4m3 codes (bytes 0,1 or 2,3 of `w`) -> packed bf16x2, exactly
// (every e4m3 value is a bf16 value); scale 1.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi_word) {
  bf16x2 v = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// Two e2m1 codes (byte `sel` of `w`: low nibble = first element) -> packed
// bf16x2, exactly; scale 1.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, v);
}

// e8m0 scale byte -> 2^(e-127) as fp32 (e in [1, 254] is a normal float;
// e = 0 gives 2^-127, built as a subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2] / [2,3,0,1],
// row_half_mirror, row_mirror, row_bcast:15, row_bcast:31.  Lanes of rows
// outside row_mask keep their own value.
enum : int {
  DPP_QUAD_1032 = 0xB1,
  DPP_QUAD_2301 = 0x4E,
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
  DPP_ROW_BCAST15 = 0x142,
  DPP_ROW_BCAST31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Sum over groups of G consecutive lanes (G = 16, 32 or 64): every lane of a
// group ends with the group's sum, bit-identical in all of them (each step
// adds two values that the partner lane adds in the other order).  Within a
// 16-lane row the moves are DPP; across rows one ds_bpermute per step.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  v += dpp_f32<DPP_QUAD_1032>(v);
  v += dpp_f32<DPP_QUAD_2301>(v);
  v += dpp_f32<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f32<DPP_ROW_MIRROR>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16, WAVE);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, WAVE);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<WAVE>(v); }

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// Arrival of the calling workgroup at a device-wide counter.  Every thread's
// global stores so far are waited for, one thread publishes them to the
// device (agent-scope release) and bumps the counter; the call returns true
// in exactly one workgroup, the one whose arrival is number `total`, and that
// workgroup then observes every other arriving workgroup's stores
// (agent-scope acquire).  wrap: the counter is bumped with atomicInc so it
// returns to 0 by itself after `total` arrivals; otherwise the caller resets
// it.  One fence per workgroup, not per thread: an agent-scope release
// writes back the XCD's whole L2.
__device__ __forceinline__ bool arrive_last(uint32_t *counter, uint32_t total, bool wrap,
                                            int *flag_lds) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have reached L2
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = wrap ? atomicInc(counter, total - 1) : atomicAdd(counter, 1u);
    const bool last = old == total - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag_lds = last;
  }
  __syncthreads();
  return *flag_lds != 0;
}

}  // namespace moe
