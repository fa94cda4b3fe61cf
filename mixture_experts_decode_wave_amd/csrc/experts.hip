// Expert kernels of the MoE decode layer:
//   gate+up pass  act[p, i]  = silu(Wg_e[i] . v) * (Wu_e[i] . v)
//   down pass     y[p, r]    = Wd_e[r] . act[p]
//   blend         out[t]     = sum_j w[t, j] * y[pos(t, j)] + g_t * y_sh[t]
// for every route p of every active expert e, plus the shared expert over
// all N rows (forward.rs: moe_expert_gate_up_shared_* then
// moe_expert_silu_down_shared_* then moe_weighted_sum_blend;
// forward_token_major.rs: the *_prefill variants over N rows).
//
// Work unit ("item") = one active expert x one tile of TR weight rows, for
// ALL routes of that expert: the tile's weights cross HBM once, however many
// tokens picked the expert.  A 256-thread workgroup walks items grid-stride.
// Inside an item the inputs of up to RG routes are staged in LDS as packed
// bf16 (fp32 for fp32 experts) in K segments; LPR lanes share a weight row,
// each lane reads its 16-byte chunks with coalesced 128-bit loads, decodes
// FP8 / MXFP4 with the gfx950 converters into bf16 pairs and accumulates
// with v_dot2_f32_bf16 in fp32; the block scale multiplies each chunk's
// partial sum.  LPR-lane butterflies reduce the row sums.  No float atomics:
// every sum has a fixed order, so results are bitwise reproducible.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int EX_THREADS = 256;
constexpr int EX_WAVES = EX_THREADS / WAVE;
constexpr int TR = 16;                 // weight rows per item
constexpr int ROWS_PER_WAVE = TR / EX_WAVES;
constexpr int LDS_BYTES = 32768;       // staged inputs

template <int FMT>
struct Lds {
  // LDS element: bf16 (2 bytes) except for fp32 experts
  static constexpr int bytes = FMT == FMT_F32 ? 4 : 2;
};

// Decoded 16-byte chunk: EPC values as packed bf16 pairs (or fp32).
template <int FMT>
struct Dec {
  static constexpr int EPC = ChunkElems<FMT>::value;
  static constexpr int WORDS = FMT == FMT_F32 ? 4 : EPC / 2;
  uint32_t v[WORDS];
};

template <int FMT>
__device__ __forceinline__ void decode(const u32x4 &raw, Dec<FMT> &d) {
  if constexpr (FMT == FMT_F32 || FMT == FMT_BF16) {
    d.v[0] = raw.x; d.v[1] = raw.y; d.v[2] = raw.z; d.v[3] = raw.w;
  } else if constexpr (FMT == FMT_FP8) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      d.v[2 * i] = fp8x2_to_bf16x2(w[i], false);
      d.v[2 * i + 1] = fp8x2_to_bf16x2(w[i], true);
    }
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      d.v[4 * i + 0] = fp4x2_to_bf16x2<0>(w[i]);
      d.v[4 * i + 1] = fp4x2_to_bf16x2<1>(w[i]);
      d.v[4 * i + 2] = fp4x2_to_bf16x2<2>(w[i]);
      d.v[4 * i + 3] = fp4x2_to_bf16x2<3>(w[i]);
    }
  }
}

// dot of a decoded chunk with the matching LDS input chunk
template <int FMT>
__device__ __forceinline__ float chunk_dot(const Dec<FMT> &d, const uint8_t *xl, float acc) {
  if constexpr (FMT == FMT_F32) {
    const f32x4 x = *(const f32x4 *)xl;
    acc = fmaf(__uint_as_float(d.v[0]), x.x, acc);
    acc = fmaf(__uint_as_float(d.v[1]), x.y, acc);
    acc = fmaf(__uint_as_float(d.v[2]), x.z, acc);
    acc = fmaf(__uint_as_float(d.v[3]), x.w, acc);
  } else {
    constexpr int Q = Dec<FMT>::WORDS / 4;  // 16-byte LDS reads
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const u32x4 x = *(const u32x4 *)(xl + 16 * q);
      acc = dot2(d.v[4 * q + 0], x.x, acc);
      acc = dot2(d.v[4 * q + 1], x.y, acc);
      acc = dot2(d.v[4 * q + 2], x.z, acc);
      acc = dot2(d.v[4 * q + 3], x.w, acc);
    }
  }
  return acc;
}

// scale of the chunk holding columns [col, col + EPC) of row `row`
template <int FMT>
__device__ __forceinline__ float chunk_scale(const void *s, int row, int col, int K) {
  if constexpr (FMT == FMT_FP8) {
    const int bc = (K + 127) >> 7;
    return ((const float *)s)[(size_t)(row >> 7) * bc + (col >> 7)];
  } else if constexpr (FMT == FMT_MXFP4) {
    return e8m0_to_f32(((const uint8_t *)s)[(size_t)row * (K >> 5) + (col >> 5)]);
  } else {
    return 1.f;
  }
}

// bytes of one weight row in storage
template <int FMT>
__device__ __forceinline__ size_t row_bytes(int K) {
  if constexpr (FMT == FMT_F32) return (size_t)K * 4;
  else if constexpr (FMT == FMT_BF16) return (size_t)K * 2;
  else if constexpr (FMT == FMT_FP8) return (size_t)K;
  else return (size_t)K / 2;
}

// Stage inputs rows [k0, k0 + kn) of `nr` vectors into LDS (row stride ks
// elements).  Source rows are fp32 or bf16.
template <int FMT, bool SRC_F32, int RG>
__device__ __forceinline__ void stage(uint8_t *lds, const void *src, const int *rows_of, int nr,
                                      int K, int k0, int kn, int ks) {
  constexpr int LB = Lds<FMT>::bytes;
  // work in 8-element groups (16 B of bf16 LDS / 32 B of fp32 LDS)
  const int groups = kn / 8;
  for (int i = threadIdx.x; i < nr * groups; i += EX_THREADS) {
    const int r = i / groups, gi = i - r * groups;
    const size_t row = (size_t)rows_of[r];
    const int col = k0 + gi * 8;
    uint8_t *dst = lds + ((size_t)r * ks + gi * 8) * LB;
    if constexpr (SRC_F32) {
      const f32x4 *p = (const f32x4 *)((const float *)src + row * K + col);
      const f32x4 a = p[0], b = p[1];
      if constexpr (LB == 4) {
        ((f32x4 *)dst)[0] = a;
        ((f32x4 *)dst)[1] = b;
      } else {
        u32x4 o;
        o.x = pack_bf16x2(a.x, a.y);
        o.y = pack_bf16x2(a.z, a.w);
        o.z = pack_bf16x2(b.x, b.y);
        o.w = pack_bf16x2(b.z, b.w);
        *(u32x4 *)dst = o;
      }
    } else {
      *(u32x4 *)dst = *(const u32x4 *)((const uint16_t *)src + row * K + col);
    }
  }
}

template <int NMAT, int RG, int RPL>
struct Acc {
  float v[NMAT][RPL][RG];
};

// One item: TR rows [row0, row0+TR) of NMAT matrices of K columns, for
// `nroute` input vectors whose source rows are given by rows_of().
template <int FMT, int NMAT, int LPR, bool SRC_F32, int RG>
__device__ void item_body(uint8_t *lds, int *rows_lds, const uint8_t *w0, const uint8_t *w1,
                          const void *s0, const void *s1, int row0, int rows, int K,
                          const void *src, const int32_t *route_map, int route_base,
                          int nroute, float *out, int out_base, bool silu_mul) {
  constexpr int EPC = ChunkElems<FMT>::value;
  constexpr int LB = Lds<FMT>::bytes;
  constexpr int RPL = TR * LPR / EX_THREADS;  // rows per lane
  constexpr int SUBS = WAVE / LPR;            // rows a wave works on at once
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int sub = lane / LPR, l = lane % LPR;
  const int ks = ((LDS_BYTES / LB) / RG) / EPC * EPC;  // staged columns per segment
  const size_t rb = row_bytes<FMT>(K);

  for (int g0 = 0; g0 < nroute; g0 += RG) {
    const int nr = min(RG, nroute - g0);
    Acc<NMAT, RG, RPL> acc;
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
      for (int q = 0; q < RPL; q++)
#pragma unroll
        for (int r = 0; r < RG; r++) acc.v[m][q][r] = 0.f;

    __syncthreads();  // previous readers of rows_lds / lds are done
    if (threadIdx.x < RG)
      rows_lds[threadIdx.x] =
          threadIdx.x < nr ? (route_map ? route_map[route_base + g0 + threadIdx.x]
                                        : route_base + g0 + (int)threadIdx.x)
                           : 0;
    for (int k0 = 0; k0 < K; k0 += ks) {
      const int kn = min(ks, K - k0);
      __syncthreads();
      stage<FMT, SRC_F32, RG>(lds, src, rows_lds, nr, K, k0, kn, ks);
      __syncthreads();
      const int cn = kn / EPC;
      const int c0 = k0 / EPC;
      for (int c = l; c < cn; c += LPR) {
        Dec<FMT> d[NMAT][RPL];
        float sc[NMAT][RPL];
#pragma unroll
        for (int q = 0; q < RPL; q++) {
          const int row = row0 + wave * ROWS_PER_WAVE + sub + SUBS * q;
#pragma unroll
          for (int m = 0; m < NMAT; m++) {
            const uint8_t *wm = m == 0 ? w0 : w1;
            const void *sm = m == 0 ? s0 : s1;
            u32x4 raw = {0, 0, 0, 0};
            sc[m][q] = 0.f;
            if (row < rows) {
              raw = __builtin_nontemporal_load((const u32x4 *)(wm + (size_t)row * rb) + c0 + c);
              sc[m][q] = chunk_scale<FMT>(sm, row, (c0 + c) * EPC, K);
            }
            decode<FMT>(raw, d[m][q]);
          }
        }
#pragma unroll
        for (int r = 0; r < RG; r++) {
          if (r < nr) {
            const uint8_t *xl = lds + ((size_t)r * ks + (size_t)c * EPC) * LB;
#pragma unroll
            for (int q = 0; q < RPL; q++)
#pragma unroll
              for (int m = 0; m < NMAT; m++) {
                if constexpr (FMT == FMT_FP8 || FMT == FMT_MXFP4)
                  acc.v[m][q][r] = fmaf(chunk_dot<FMT>(d[m][q], xl, 0.f), sc[m][q], acc.v[m][q][r]);
                else
                  acc.v[m][q][r] = chunk_dot<FMT>(d[m][q], xl, acc.v[m][q][r]);
              }
          }
        }
      }
    }
    // reduce over the LPR lanes of a row and write
#pragma unroll
    for (int q = 0; q < RPL; q++) {
      const int row = row0 + wave * ROWS_PER_WAVE + sub + SUBS * q;
#pragma unroll
      for (int r = 0; r < RG; r++) {
        float v0 = group_sum<LPR>(acc.v[0][q][r]);
        float res = v0;
        if constexpr (NMAT == 2) {
          const float v1 = group_sum<LPR>(acc.v[1][q][r]);
          res = silu_mul ? v0 * sigmoidf_(v0) * v1 : v0;
        }
        if (l == r && r < nr && row < rows) out[(size_t)(out_base + g0 + r) * rows + row] = res;
      }
    }
  }
}

template <int FMT, int NMAT, int LPR, bool SRC_F32>
__global__ __launch_bounds__(EX_THREADS) void expert_gemv_kernel(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int rows_lds[8];
  const int n_items = a.sh_items + min(*a.n_active, a.max_active) * a.tiles;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const uint8_t *w0, *w1 = nullptr;
    const void *s0, *s1 = nullptr;
    int row0, rows, K, nroute, route_base, out_base;
    const void *src;
    const int32_t *route_map;
    float *out;
    if (item < a.sh_items) {
      w0 = (const uint8_t *)a.sh_w0;
      s0 = a.sh_s0;
      if (NMAT == 2) { w1 = (const uint8_t *)a.sh_w1; s1 = a.sh_s1; }
      row0 = item * TR;
      rows = a.sh_rows;
      K = a.sh_K;
      nroute = a.N;
      route_base = 0;
      route_map = nullptr;  // input row t for t < N
      src = a.sh_src;
      out = a.sh_out;
      out_base = 0;
    } else {
      const int it = item - a.sh_items;
      const int slot = it / a.tiles;
      const int e = a.active[slot];
      w0 = (const uint8_t *)a.w0[e];
      s0 = a.s0 ? a.s0[e] : nullptr;
      if (NMAT == 2) { w1 = (const uint8_t *)a.w1[e]; s1 = a.s1 ? a.s1[e] : nullptr; }
      row0 = (it - slot * a.tiles) * TR;
      rows = a.rows;
      K = a.K;
      route_base = a.off[slot];
      nroute = a.off[slot + 1] - route_base;
      route_map = a.src_by_token ? a.route_tok : nullptr;
      src = a.src;
      out = a.out;
      out_base = route_base;
      // without a token map the input row is the route position itself
    }
    if (nroute <= 1)
      item_body<FMT, NMAT, LPR, SRC_F32, 1>(lds, rows_lds, w0, w1, s0, s1, row0, rows, K, src,
                                            route_map, route_base, nroute, out, out_base, NMAT == 2);
    else if (nroute <= 2)
      item_body<FMT, NMAT, LPR, SRC_F32, 2>(lds, rows_lds, w0, w1, s0, s1, row0, rows, K, src,
                                            route_map, route_base, nroute, out, out_base, NMAT == 2);
    else if (nroute <= 4)
      item_body<FMT, NMAT, LPR, SRC_F32, 4>(lds, rows_lds, w0, w1, s0, s1, row0, rows, K, src,
                                            route_map, route_base, nroute, out, out_base, NMAT == 2);
    else
      item_body<FMT, NMAT, LPR, SRC_F32, 8>(lds, rows_lds, w0, w1, s0, s1, row0, rows, K, src,
                                            route_map, route_base, nroute, out, out_base, NMAT == 2);
  }
}

template <int FMT, int NMAT, bool SRC_F32>
hipError_t launch_lpr(int lpr, const GemvArgs &a, int grid, hipStream_t s) {
  switch (lpr) {
    case 16:
      hipLaunchKernelGGL((expert_gemv_kernel<FMT, NMAT, 16, SRC_F32>), dim3(grid),
                         dim3(EX_THREADS), 0, s, a);
      break;
    case 32:
      hipLaunchKernelGGL((expert_gemv_kernel<FMT, NMAT, 32, SRC_F32>), dim3(grid),
                         dim3(EX_THREADS), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((expert_gemv_kernel<FMT, NMAT, 64, SRC_F32>), dim3(grid),
                         dim3(EX_THREADS), 0, s, a);
      break;
  }
  return hipGetLastError();
}

// lanes per weight row: enough chunks per lane to keep loads in flight
int pick_lpr(int K, int epc) {
  const int C = K / epc;
  if (C >= 4 * 64) return 64;
  if (C >= 4 * 32) return 32;
  return 16;
}

constexpr int MAX_GRID = 2048;

// ---------------------------------------------------------------- blend

template <bool F32>
__global__ __launch_bounds__(256) void blend_kernel(BlendArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  float g = 1.f;
  if (a.y_sh && a.gate_vec) {
    float d = 0.f;
    for (int i = threadIdx.x; i < a.h; i += 256) {
      float xv, gv;
      if constexpr (F32) {
        xv = ((const float *)a.x)[(size_t)t * a.h + i];
        gv = ((const float *)a.gate_vec)[i];
      } else {
        xv = __uint_as_float((uint32_t)((const uint16_t *)a.x)[(size_t)t * a.h + i] << 16);
        gv = __uint_as_float((uint32_t)((const uint16_t *)a.gate_vec)[i] << 16);
      }
      d = fmaf(xv, gv, d);
    }
    d = wave_sum(d);
    if (threadIdx.x % WAVE == 0) red[threadIdx.x / WAVE] = d;
    __syncthreads();
    g = sigmoidf_(red[0] + red[1] + red[2] + red[3]);
  }
  if (c >= a.h) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.k; j++) {
    const int p = a.route_pos[(size_t)t * a.k + j];
    if (p >= 0) {
      const float wj = a.w[(size_t)t * a.k + j];
      const f32x4 yv = *(const f32x4 *)(a.y + (size_t)p * a.h + c);
      acc.x = fmaf(wj, yv.x, acc.x);
      acc.y = fmaf(wj, yv.y, acc.y);
      acc.z = fmaf(wj, yv.z, acc.z);
      acc.w = fmaf(wj, yv.w, acc.w);
    }
  }
  if (a.y_sh) {
    const f32x4 yv = *(const f32x4 *)(a.y_sh + (size_t)t * a.h + c);
    acc.x = fmaf(g, yv.x, acc.x);
    acc.y = fmaf(g, yv.y, acc.y);
    acc.z = fmaf(g, yv.z, acc.z);
    acc.w = fmaf(g, yv.w, acc.w);
  }
  if constexpr (F32) {
    *(f32x4 *)((float *)a.out + (size_t)t * a.h + c) = acc;
  } else {
    u32x2 o;
    o.x = pack_bf16x2(acc.x, acc.y);
    o.y = pack_bf16x2(acc.z, acc.w);
    *(u32x2 *)((uint16_t *)a.out + (size_t)t * a.h + c) = o;
  }
}

}  // namespace

hipError_t launch_expert_gemv(int fmt, int nmat, bool src_f32, const GemvArgs &a, int max_items,
                              hipStream_t s) {
  const int grid = max_items < MAX_GRID ? (max_items > 0 ? max_items : 1) : MAX_GRID;
  const int epc = fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 8 : fmt == FMT_FP8 ? 16 : 32;
  const int lpr = pick_lpr(a.K, epc);
#define MOE_DISPATCH(F)                                                              \
  if (nmat == 2)                                                                     \
    return src_f32 ? launch_lpr<F, 2, true>(lpr, a, grid, s)                         \
                   : launch_lpr<F, 2, false>(lpr, a, grid, s);                       \
  return launch_lpr<F, 1, true>(lpr, a, grid, s);
  switch (fmt) {
    case FMT_F32: {
      MOE_DISPATCH(FMT_F32)
    }
    case FMT_BF16: {
      MOE_DISPATCH(FMT_BF16)
    }
    case FMT_FP8: {
      MOE_DISPATCH(FMT_FP8)
    }
    default: {
      MOE_DISPATCH(FMT_MXFP4)
    }
  }
#undef MOE_DISPATCH
}

hipError_t launch_blend(bool act_f32, const BlendArgs &a, hipStream_t s) {
  dim3 grid((a.h + 1023) / 1024, a.N), block(256);
  if (act_f32)
    hipLaunchKernelGGL(blend_kernel<true>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(blend_kernel<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
