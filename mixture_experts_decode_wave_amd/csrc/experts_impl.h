// Expert kernels of the MoE decode layer:
//   gate+up pass  act[p, i]  = silu(Wg_e[i] . v) * (Wu_e[i] . v)
//   down pass     y[p, r]    = Wd_e[r] . act[p]
// for every route p of every active expert e, plus the shared expert over
// all N rows (forward.rs: moe_expert_gate_up_shared_* then
// moe_expert_silu_down_shared_* then moe_weighted_sum_blend;
// forward_token_major.rs: the *_prefill variants over N rows).
//
// Work unit ("item") = one active expert x one tile of TR weight rows, for
// ALL routes of that expert: the tile's weights cross HBM once, however many
// tokens picked the expert.  A 256-thread workgroup walks items grid-stride.
//
// Weights are stored in 16-row x 64-byte tiles (tile_off below), so both
// inner products read them a whole 1 KB tile per wave-wide 16-byte load,
// with non-temporal loads: contiguous blocks stream from HBM far better than
// 16 rows' 64-byte pieces 1-2 KB apart, and the stream does not evict the
// staged input rows from L2.
//
// Two inner products, chosen per item from its route count R:
//  * R <= 4 (decode: one or a few tokens per expert) -- VALU GEMV.  A wave
//    reads 16 rows a tile at a time, lane (row l/4, piece l%4); the loads
//    run D tiles deep (the first are issued before the inputs are staged, so
//    HBM latency overlaps the LDS fill); FP8 / MXFP4 chunks are decoded by
//    the gfx950 converters into bf16 pairs and accumulated with
//    v_dot2_f32_bf16 in fp32; the block scale multiplies each chunk's
//    partial sum; quad butterflies and 4 K parts in a fixed order reduce.
//  * R > 4 (verify batches, shared expert at larger N) -- MFMA.  A wave owns
//    16 weight rows; lane (row = l%16, kg = l/16) decodes piece kg of a tile
//    per k-step and feeds v_mfma_f32_16x16x32_bf16 with the routes' inputs
//    (16 per pass) as the N operand, read from LDS.
//
// No float atomics: every sum has a fixed order, so the results are bitwise
// reproducible from run to run.
#pragma once

#include <climits>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int EX_THREADS = 256;
constexpr int EX_WAVES = EX_THREADS / WAVE;
constexpr int XPAD = 16;      // bytes of padding per staged row (LDS bank spread)
constexpr int VALU_SB = 2;    // staging loads in flight per thread, VALU path
constexpr int MFMA_SB = 8;    // and MFMA path
constexpr int MFMA_D = 4;     // MFMA path: k-steps of weight loads in flight per wave
constexpr int ROWS_OUT = 64;  // rows_lds: input rows at [0, RG), output rows at [ROWS_OUT, +RG)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int FMT>
struct Lds {
  static constexpr int bytes = FMT == FMT_F32 ? 4 : 2;  // bf16 except for fp32 experts
};

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

// MXFP4 chunk with its power-of-two block scale folded into the bf16 values
// (exact: every e2m1 value times 2^k with a normal result is a bf16 value)
__device__ __forceinline__ void decode_scaled_fp4(const u32x4 &raw, float scale, Dec<FMT_MXFP4> &d) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    d.v[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0));
    d.v[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1));
    d.v[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2));
    d.v[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3));
  }
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// The 8 bf16 values (as 4 words) of MFMA j of a chunk, the j-th eighth of the
// decode above: MXFP4 word j, FP8 words 2j and 2j+1, BF16 the chunk itself.
template <int FMT, int J>
__device__ __forceinline__ u32x4 decode_part(const u32x4 &raw, float scale) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (FMT == FMT_MXFP4) {
    return u32x4{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[J], scale, 0)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[J], scale, 1)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[J], scale, 2)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[J], scale, 3))};
  } else if constexpr (FMT == FMT_FP8) {
    return u32x4{fp8x2_to_bf16x2(w[2 * J], false), fp8x2_to_bf16x2(w[2 * J], true),
                 fp8x2_to_bf16x2(w[2 * J + 1], false), fp8x2_to_bf16x2(w[2 * J + 1], true)};
  } else {
    static_assert(FMT == FMT_BF16 && J == 0, "one MFMA a bf16 chunk");
    return raw;
  }
}

template <int FMT>
__device__ __forceinline__ float chunk_dot(const Dec<FMT> &d, const uint8_t *xl, float acc) {
  if constexpr (FMT == FMT_F32) {
    const f32x4 x = *(const f32x4 *)xl;
    acc = fmaf(__uint_as_float(d.v[0]), x.x, acc);
    acc = fmaf(__uint_as_float(d.v[1]), x.y, acc);
    acc = fmaf(__uint_as_float(d.v[2]), x.z, acc);
    acc = fmaf(__uint_as_float(d.v[3]), x.w, acc);
  } else {
    constexpr int Q = Dec<FMT>::WORDS / 4;
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

// dot of a decoded chunk with an input chunk held in registers (same layout)
template <int FMT>
__device__ __forceinline__ float chunk_dot_regs(const Dec<FMT> &d, const uint32_t *x, float acc) {
  if constexpr (FMT == FMT_F32) {
#pragma unroll
    for (int i = 0; i < 4; i++) acc = fmaf(__uint_as_float(d.v[i]), __uint_as_float(x[i]), acc);
  } else {
#pragma unroll
    for (int i = 0; i < Dec<FMT>::WORDS; i++) acc = dot2(d.v[i], x[i], acc);
  }
  return acc;
}

template <int FMT>
__device__ __forceinline__ size_t row_bytes(int K) {
  if constexpr (FMT == FMT_F32) return (size_t)K * 4;
  else if constexpr (FMT == FMT_BF16) return (size_t)K * 2;
  else if constexpr (FMT == FMT_FP8) return (size_t)K;
  else return (size_t)K / 2;
}

// Quotient by a divisor d >= 2 known per segment, as a multiply-high by
// m = ceil(2^32 / d): floor(i m / 2^32) = floor(i / d) whenever
// i (m d - 2^32) < 2^32, which holds for i < 2^17 and d <= 2^15 (m d - 2^32 < d).
// The staging loops below split flat indices i < 2^17 into (row, piece) this
// way instead of by an integer division per element.
struct FastDiv {
  uint32_t d, m;
};
__device__ __forceinline__ FastDiv fast_div(uint32_t d) { return {d, 0xFFFFFFFFu / d + 1u}; }
__device__ __forceinline__ uint32_t quot(uint32_t i, FastDiv f) { return __umulhi(i, f.m); }

// Stage columns [k0, k0 + kn) of `nr` input rows into LDS, row stride
// `stride` bytes.  Each thread first loads up to SB 8-element groups (fp32 or
// bf16 in memory), then stores them (as bf16, or fp32 for fp32 layers), so a
// thread keeps SB loads in flight instead of one.
template <int FMT, bool SRC_F32, int SB>
__device__ __forceinline__ void stage(uint8_t *lds, const void *src, const int *rows_of, int nr,
                                      int K, int k0, int kn, int stride) {
  constexpr int LB = Lds<FMT>::bytes;
  const int groups = kn / 8;  // 8-element groups per row (>= 4)
  const int total = nr * groups;
  const FastDiv gdiv = fast_div(groups);
  for (int i0 = threadIdx.x; i0 < total; i0 += EX_THREADS * SB) {
    f32x4 va[SB], vb[SB];
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = i0 + u * EX_THREADS;
      va[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      vb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < total) {
        const int r = quot(i, gdiv), gi = i - r * groups;
        const size_t row = (size_t)rows_of[r];
        const int col = k0 + gi * 8;
        if constexpr (SRC_F32) {
          const f32x4 *p = (const f32x4 *)((const float *)src + row * K + col);
          va[u] = p[0];
          vb[u] = p[1];
        } else {
          va[u] = __builtin_bit_cast(f32x4, *(const u32x4 *)((const uint16_t *)src + row * K + col));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = i0 + u * EX_THREADS;
      if (i < total) {
        const int r = quot(i, gdiv), gi = i - r * groups;
        uint8_t *dst = lds + (size_t)r * stride + (size_t)gi * 8 * LB;
        if constexpr (SRC_F32 && LB == 4) {
          ((f32x4 *)dst)[0] = va[u];
          ((f32x4 *)dst)[1] = vb[u];
        } else if constexpr (SRC_F32) {
          u32x4 o;
          o.x = pack_bf16x2(va[u].x, va[u].y);
          o.y = pack_bf16x2(va[u].z, va[u].w);
          o.z = pack_bf16x2(vb[u].x, vb[u].y);
          o.w = pack_bf16x2(vb[u].z, vb[u].w);
          *(u32x4 *)dst = o;
        } else {
          *(u32x4 *)dst = __builtin_bit_cast(u32x4, va[u]);
        }
      }
    }
  }
}

// Columns per staged segment: at most `cap` (what the LDS holds), a multiple
// of `unit`, and the K columns split into equal segments rather than full
// ones and a short remainder (each segment costs a staging round).
__device__ __forceinline__ int even_segment(int K, int cap, int unit) {
  const int most = cap / unit * unit;
  const int nseg = (K + most - 1) / most;
  const int per = (K + nseg - 1) / nseg;
  return (per + unit - 1) / unit * unit;
}

// What one item works on.
struct Item {
  const uint8_t *w[2];  // weight matrices (NMAT of them)
  const void *s[2];     // their scales
  int row0, rows, K;    // rows [row0, row0 + TR) of a rows x K matrix
  const void *src;      // inputs
  const int32_t *route_map;  // input row of route position p (NULL: p itself)
  int route_base, nroute;    // route positions [route_base, route_base + nroute)
  const int32_t *out_map;    // output row of route position p (NULL: p itself)
  void *out;                 // out[out row of route_base + r][row], rows wide
  int npass;                 // MFMA path: passes of TR rows, from row0 on
};

// Output element of a pass: the gate+up pass stores act in bf16 (the down
// pass reads it as bf16 anyway), fp32 experts and the down pass store fp32.
template <int FMT, int NMAT>
__device__ __forceinline__ void store_out(void *out, size_t i, float v) {
  if constexpr (NMAT == 2 && FMT != FMT_F32)
    ((uint16_t *)out)[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    ((float *)out)[i] = v;
}

// Rows of routes g0 .. g0+RG-1: their input rows into rows_lds[0..RG) and
// their output rows into rows_lds[ROWS_OUT..ROWS_OUT+RG) (0 beyond nr).
template <int RG>
__device__ __forceinline__ void route_rows(int *rows_lds, const Item &it, int g0, int nr) {
  if (threadIdx.x < RG) {
    const int r = threadIdx.x, p = it.route_base + g0 + r;
    const bool ok = r < nr;
    rows_lds[r] = ok ? (it.route_map ? it.route_map[p] : p) : 0;
    rows_lds[ROWS_OUT + r] = ok ? (it.out_map ? it.out_map[p] : p) : 0;
  }
}

// FP8 block scales of the item's NB 128-row blocks from row0 (row0 a multiple
// of 128, or NB == 1 and the pass within one block), all column blocks, per
// matrix: block rb of matrix m into slot m NB + rb; a block past the matrix is
// not read.
template <int FMT, int NMAT, int NB = 1, int NT = EX_THREADS>
__device__ __forceinline__ void stage_scales(float *s_lds, const Item &it, int row0) {
  if constexpr (FMT == FMT_FP8) {
    const int bc = (it.K + 127) >> 7;
    const int nrb = min(NB, (it.rows - row0 + 127) >> 7);
    for (int i = threadIdx.x; i < NMAT * NB * bc; i += NT) {
      const int q = i / bc, b = i - q * bc;  // slot, column block
      const int m = q / NB, rb = q - m * NB;
      if (rb < nrb) {
        const float *sm = (const float *)(m == 0 ? it.s[0] : it.s[1]);  // no dynamic index
        s_lds[q * 128 + b] = sm[(size_t)((row0 >> 7) + rb) * bc + b];
      }
    }
  }
}

// ------------------------------------------------------------------ tiled weight layout

// Expert weights are stored in tiles of 16 rows x 64 bytes.  The rows of a
// matrix come in groups of 16; a row group is 16 rb contiguous bytes (rb the
// bytes of one row), in which tile column t holds bytes [64 t, 64 t + 64) of
// the group's 16 rows, row after row (1 KB), tile columns in order.  When rb
// is not a multiple of 64 the last tile column is narrower (16 x (rb % 64)).
// A 16-byte chunk c of a row is piece c % 4 of tile column c / 4, so one
// 16-byte load per lane reads a whole 1 KB tile: 16 rows x 4 lanes.
__device__ __forceinline__ size_t tile_off(int row, int c, size_t rb) {
  const int full = (int)(rb >> 6);
  const int t = c >> 2;
  const int wid = t < full ? 64 : (int)(rb & 63);
  return (size_t)(row >> 4) * 16 * rb + (size_t)t * 1024 + (size_t)(row & 15) * wid +
         (size_t)(c & 3) * 16;
}

// Lane sum over the 4 lanes of a row (consecutive lanes): (v0 + v1) + (v2 + v3)
// in every lane, bit-identical in all four (each step adds two values that
// the partner lane adds in the other order).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f32<DPP_QUAD_1032>(v);
  v += dpp_f32<DPP_QUAD_2301>(v);
  return v;
}

// ------------------------------------------------------------------ VALU path
//
// A wave reads one row block (16 rows) a tile column (1 KB) per load: lane l
// holds row l / 4 of the block and piece q = l % 4 of the tile, i.e. chunk
// c = 4 j + q of tile column j.  Tile columns are dealt to 4 K parts, part
// p = j % 4.  Every (row, route) sum is built the same way whatever the tile
// size and the route group: each lane sums its chunks of part p in ascending
// j (one fp32 partial per part), the 4 lanes of a row are summed by
// quad_sum, then the parts are added in order ((p0 + p1) + p2) + p3.  So a
// route's result does not depend on the item shape or on the other routes.
//   TR = 64: wave w owns row block w and all 4 parts (a load stream over
//            every tile column, partial j % 4);
//   TR = 16: the 4 waves share the one row block, wave w taking part w; the
//            parts meet in LDS.
constexpr int VPARTS = 4;
constexpr int VALU_D = 4;  // tile columns of weight loads in flight per wave

template <int FMT, int NMAT>
struct VBatch {
  u32x4 raw[NMAT];
  uint32_t sb[NMAT];  // MXFP4 scale bytes
};

template <int FMT, int NMAT, int TR, bool SRC_F32, int RG>
__device__ __forceinline__ void valu_item(uint8_t *lds, int lds_bytes, float *s_lds, int *rows_lds,
                                          float *vred, const Item &it) {
  constexpr int EPC = ChunkElems<FMT>::value;
  constexpr int LB = Lds<FMT>::bytes;
  constexpr int NB = TR / 16;                 // row blocks of the item
  static_assert(NB == 1 || NB == 4, "VALU items are 16 or 64 rows");
  constexpr int PP = NB == 4 ? VPARTS : 1;    // K parts a wave sums
  constexpr int JS = NB == 4 ? 1 : VPARTS;    // tile-column stride of a wave
  constexpr int D = VALU_D;
  static_assert(D % VPARTS == 0, "a ring of whole part cycles");
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int m = lane >> 2, q = lane & 3;
  const int part = NB == 4 ? 0 : wave;        // NB == 1: the wave's part
  const int row = it.row0 + (NB == 4 ? wave * 16 : 0) + m;
  const bool row_ok = row < it.rows;
  const size_t rb = row_bytes<FMT>(it.K);
  const int cn = it.K / EPC;                  // chunks per row
  // staged columns per segment: whole tile columns (4 chunks)
  const int KS = even_segment(it.K, ((lds_bytes / RG) - XPAD) / LB, 4 * EPC);
  const int STRIDE = KS * LB + XPAD;

  for (int g0 = 0; g0 < it.nroute; g0 += RG) {
    const int nr = min(RG, it.nroute - g0);
    float acc[NMAT][PP][RG];
#pragma unroll
    for (int mm = 0; mm < NMAT; mm++)
#pragma unroll
      for (int p = 0; p < PP; p++)
#pragma unroll
        for (int r = 0; r < RG; r++) acc[mm][p][r] = 0.f;

    for (int k0 = 0; k0 < it.K; k0 += KS) {
      const int kn = min(KS, it.K - k0);
      const int c0 = k0 / EPC;                // first chunk of the segment (a multiple of 4)
      const int j0 = c0 >> 2, j1 = (c0 + kn / EPC + 3) >> 2;
      // this wave's tile columns of the segment: j = jf, jf + JS, ... < j1
      const int jf = NB == 4 ? j0 : j0 + ((part - j0) % VPARTS + VPARTS) % VPARTS;
      const int ns = jf < j1 ? (j1 - jf + JS - 1) / JS : 0;

      auto load = [&](VBatch<FMT, NMAT> &b, int i) {
        const int c = 4 * (jf + JS * i) + q;
#pragma unroll
        for (int mm = 0; mm < NMAT; mm++) {
          b.raw[mm] = u32x4{0, 0, 0, 0};
          b.sb[mm] = 127;
          if (i < ns && c < cn && row_ok) {
            b.raw[mm] = __builtin_nontemporal_load((const u32x4 *)(it.w[mm] + tile_off(row, c, rb)));
            if constexpr (FMT == FMT_MXFP4)
              b.sb[mm] = ((const uint8_t *)it.s[mm])[(size_t)row * (it.K >> 5) + c];
          }
        }
      };

      VBatch<FMT, NMAT> buf[D];
#pragma unroll
      for (int d = 0; d < D; d++) load(buf[d], d);  // in flight during the staging below

      __syncthreads();  // previous readers of the LDS are done
      if (g0 == 0 && k0 == 0) stage_scales<FMT, NMAT>(s_lds, it, it.row0);
      route_rows<RG>(rows_lds, it, g0, nr);
      __syncthreads();
      stage<FMT, SRC_F32, VALU_SB>(lds, it.src, rows_lds, nr, it.K, k0, kn, STRIDE);
      __syncthreads();

      for (int i0 = 0; i0 < ns; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
          const int i = i0 + d;
          if (i < ns) {
            const int c = 4 * (jf + JS * i) + q;
            // part of this tile column: (j0 + i) % 4 = d % 4 for TR = 64 (j0
            // and i0 are multiples of 4), the wave's part for TR = 16
            const int pi = NB == 4 ? (d % VPARTS) : 0;
            if (c < cn) {
              // this chunk of every staged input row, then each decoded weight
              // chunk against all of them
              uint32_t xr[RG][Dec<FMT>::WORDS];
#pragma unroll
              for (int r = 0; r < RG; r++) {
                if (r < nr) {
                  const uint8_t *xl = lds + (size_t)r * STRIDE + (size_t)(c - c0) * EPC * LB;
#pragma unroll
                  for (int w4 = 0; w4 < Dec<FMT>::WORDS; w4 += 4) {
                    const u32x4 xv = *(const u32x4 *)(xl + 4 * w4);
                    xr[r][w4] = xv.x;
                    xr[r][w4 + 1] = xv.y;
                    xr[r][w4 + 2] = xv.z;
                    xr[r][w4 + 3] = xv.w;
                  }
                }
              }
#pragma unroll
              for (int mm = 0; mm < NMAT; mm++) {
                Dec<FMT> dec;
                decode<FMT>(buf[d].raw[mm], dec);
                float sc = 1.f;
                if constexpr (FMT == FMT_FP8)
                  sc = s_lds[mm * 128 + ((c * EPC) >> 7)];
                else if constexpr (FMT == FMT_MXFP4)
                  sc = e8m0_to_f32(buf[d].sb[mm]);
#pragma unroll
                for (int p = 0; p < PP; p++) {
                  if (p == pi) {
#pragma unroll
                    for (int r = 0; r < RG; r++) {
                      if (r < nr) {
                        if constexpr (FMT == FMT_FP8 || FMT == FMT_MXFP4)
                          acc[mm][p][r] =
                              fmaf(chunk_dot_regs<FMT>(dec, xr[r], 0.f), sc, acc[mm][p][r]);
                        else
                          acc[mm][p][r] = chunk_dot_regs<FMT>(dec, xr[r], acc[mm][p][r]);
                      }
                    }
                  }
                }
              }
            }
            load(buf[d], i + D);
          }
        }
      }
    }

    // lane sums, then the parts in order
    float res[RG];
    if constexpr (NB == 4) {
#pragma unroll
      for (int r = 0; r < RG; r++) {
        float v[NMAT];
#pragma unroll
        for (int mm = 0; mm < NMAT; mm++)
          v[mm] = ((quad_sum(acc[mm][0][r]) + quad_sum(acc[mm][1][r])) +
                   quad_sum(acc[mm][2][r])) + quad_sum(acc[mm][3][r]);
        res[r] = NMAT == 2 ? v[0] * sigmoidf_(v[0]) * v[NMAT - 1] : v[0];
      }
    } else {
      // vred[part][row][mat][route]
#pragma unroll
      for (int mm = 0; mm < NMAT; mm++)
#pragma unroll
        for (int r = 0; r < RG; r++) {
          const float v = quad_sum(acc[mm][0][r]);
          if (q == 0) vred[((wave * 16 + m) * NMAT + mm) * RG + r] = v;
        }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < RG; r++) {
        float v[NMAT];
#pragma unroll
        for (int mm = 0; mm < NMAT; mm++) {
          float t = vred[((0 * 16 + m) * NMAT + mm) * RG + r];
#pragma unroll
          for (int p = 1; p < VPARTS; p++) t += vred[((p * 16 + m) * NMAT + mm) * RG + r];
          v[mm] = t;
        }
        res[r] = NMAT == 2 ? v[0] * sigmoidf_(v[0]) * v[NMAT - 1] : v[0];
      }
    }
    // lane q of a row stores route q (NB == 1: wave 0 only)
#pragma unroll
    for (int r = 0; r < RG; r++) {
      if (q == r && r < nr && row_ok && (NB == 4 || wave == 0))
        store_out<FMT, NMAT>(it.out, (size_t)rows_lds[ROWS_OUT + r] * it.rows + row, res[r]);
    }
  }
}

// ------------------------------------------------------------------ MFMA path

// One staged segment of the MFMA path: columns [k0, k0 + kn) of the nr bf16
// input rows (row stride `stride` bytes) and, for MXFP4, the tile's e8m0
// scale rows of those columns (NMAT x TR rows, `sst` bytes apart, 16-byte
// pieces, zeros past the matrix).  EARLY: the thread's first SB row groups
// and first SP scale pieces are loaded into registers together and stored
// only after the barrier that frees the LDS (`bar`), so their memory round
// trip overlaps the wait for the other waves; the rest follow in rounds of
// SB.  Otherwise (the caller has passed that barrier) the rows go in rounds
// of SB, then the scale pieces.  MI355X measured the early form faster for
// the gate+up pass and slower for the down pass.
template <int FMT, int NMAT, int TR, int SB, bool EARLY, int NT = EX_THREADS>
__device__ __forceinline__ void stage_segment(uint8_t *lds, uint8_t *sc, int sst, const Item &it,
                                              const int *rows_of, int nr, int k0, int kn,
                                              int stride, bool bar, int p0, int np) {
  constexpr int SP = 4;
  constexpr int SCP = FMT == FMT_MXFP4 ? NMAT * TR : 0;  // scale rows of a pass
  const int SCB = SCP * np;                              // of the np passes from p0
  const int groups = kn / 8;  // 8-element groups per input row (>= 4)
  const int total = nr * groups;
  const int pieces = kn / 512;  // 16-byte scale pieces per scale row
  const int stot = SCB * pieces;
  const FastDiv gdiv = fast_div(groups);
  const FastDiv pdiv = fast_div(pieces > 1 ? pieces : 2);
  auto xsrc = [&](int i) {
    const int r = quot(i, gdiv), gi = i - r * groups;
    return (const u32x4 *)((const uint16_t *)it.src + (size_t)rows_of[r] * it.K + k0 + gi * 8);
  };
  auto xdst = [&](int i) {
    const int r = quot(i, gdiv), gi = i - r * groups;
    return (u32x4 *)(lds + (size_t)r * stride + (size_t)gi * 16);
  };
  auto srow = [&](int q) { return pieces > 1 ? (int)quot(q, pdiv) : q; };
  auto spiece = [&](int q) {
    const int sr = srow(q), pc = q - sr * pieces;
    const int pi = sr / SCP, rm = sr - pi * SCP;  // pass, then matrix and row within it
    const int m = rm / TR, r = rm - m * TR;
    const int row = it.row0 + TR * (p0 + pi) + r;
    u32x4 v = {0, 0, 0, 0};
    if (row < it.rows)
      v = *(const u32x4 *)((const uint8_t *)(m == 0 ? it.s[0] : it.s[1]) +
                           (size_t)row * (it.K >> 5) + (k0 >> 5) + pc * 16);
    return v;
  };
  auto sdst = [&](int q) {
    const int sr = srow(q), pc = q - sr * pieces;
    return (u32x4 *)(sc + (size_t)sr * sst + pc * 16);
  };
  u32x4 xv[SB];
  if constexpr (EARLY) {
    u32x4 sv[SP];
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = threadIdx.x + u * NT;
      xv[u] = i < total ? *xsrc(i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < SP; u++) {
      const int q = threadIdx.x + u * NT;
      sv[u] = q < stot ? spiece(q) : u32x4{0, 0, 0, 0};
    }
    if (bar) __syncthreads();
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = threadIdx.x + u * NT;
      if (i < total) *xdst(i) = xv[u];
    }
#pragma unroll
    for (int u = 0; u < SP; u++) {
      const int q = threadIdx.x + u * NT;
      if (q < stot) *sdst(q) = sv[u];
    }
  }
  constexpr int X0 = EARLY ? SB : 0;  // row groups and scale pieces already staged
  constexpr int S0 = EARLY ? SP : 0;
  for (int i0 = threadIdx.x + X0 * NT; i0 < total; i0 += SB * NT) {
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = i0 + u * NT;
      xv[u] = i < total ? *xsrc(i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int i = i0 + u * NT;
      if (i < total) *xdst(i) = xv[u];
    }
  }
  for (int q = threadIdx.x + S0 * NT; q < stot; q += NT) *sdst(q) = spiece(q);
}

// Launch shape of the MFMA path (see mfma_item) of a pass with NMAT matrices.
template <int FMT, int NMAT, int TR, int RB, int MR = 1, int NW = EX_WAVES>
struct MfmaShape {
  static constexpr int RGRP = TR / 16;             // row groups
  static constexpr int KSPLIT = NW / RGRP;         // k-splits per row group (NW waves)
  // MXFP4 with one k-split: segments are whole multiples of 512 columns, 4
  // k-steps of a wave, so with 4 k-steps in flight the weight loads run on
  // from one segment into the next -- and from an item's last segment into
  // its next route group or the workgroup's next item: the last iterations
  // load the successor's first k-steps into the slots it starts from, and the
  // stream does not drain while the next inputs are staged
  static constexpr bool CHAIN = FMT == FMT_MXFP4 && KSPLIT == 1;
  // into the next item too: the gate+up pass with 16-route groups only (the
  // down pass measured far slower chained into its next item, with the next
  // descriptor read from memory or from an LDS table alike; the wide form
  // would spill registers)
  static constexpr bool XCHAIN = CHAIN && RB == 1 && MR == 1 && NMAT == 2;
  // k-steps in flight; a 512-column MXFP4 segment is 4 k-steps of a wave,
  // and chained loads need D to divide that (MR row groups: MR times the
  // loads a k-step, so fewer k-steps)
  static constexpr int D = MR > 1 ? MFMA_D / 2 : MFMA_D;
  static_assert(!CHAIN || 4 % D == 0, "chained segments hold whole rings of k-steps");
};

// 16 weight rows x 16 RB routes per wave; TR / 16 row groups share the
// workgroup's 4 waves with 64 / TR k-splits (partials summed through LDS).
// RB > 1 (route groups of 16 RB: the grouped-GEMM shape of large steps) uses
// each decoded weight fragment for RB 16-route MFMA blocks.  MR > 1 (that
// shape too): the item's first MR passes of TR rows run at once, each wave
// holding its row group in every one of them, so each staged input fragment
// read from the LDS serves MR weight fragments.
// raw: the ring of k-steps in flight; pre: it already holds this item's
// first D k-steps; nxt (XCHAIN shapes, when has_nxt): the workgroup's next
// item, an MFMA item of the same K, whose first D k-steps the last iterations
// load.  Returns whether they did.  (The item is taken by value with a flag:
// a nullable pointer to it would keep it in scratch memory.)
template <int FMT, int NMAT, int TR, bool SRC_F32, int RB = 1, int MR = 1, int NW = EX_WAVES>
__device__ __forceinline__ bool mfma_item(uint8_t *lds, int lds_bytes, float *s_lds, int *rows_lds,
                                          const Item &it,
                                          u32x4 (&raw)[MfmaShape<FMT, NMAT, TR, RB, MR, NW>::D][NMAT * MR],
                                          bool pre, const Item &nxt, bool has_nxt) {
  static_assert(FMT != FMT_F32, "fp32 experts use the VALU path");
  constexpr int EPC = ChunkElems<FMT>::value;  // elements per lane per k-step
  constexpr int KSTEP = 4 * EPC;               // columns per k-step of a wave
  constexpr int JM = EPC / 8;                  // MFMAs per k-step and route block
  constexpr int RG = 16 * RB;
  constexpr int RGRP = TR / 16;                // row groups
  constexpr int KSPLIT = NW / RGRP;            // k-splits per row group
  constexpr int NT = NW * WAVE;                // threads of the workgroup
  static_assert(RGRP >= 1 && RGRP * KSPLIT == NW, "tile shape");
  static_assert(RB == 1 || KSPLIT == 1, "wide route groups without k-splits");
  static_assert(RG <= ROWS_OUT, "route table");
  static_assert(MR == 1 || KSPLIT == 1, "several row groups a wave without k-splits");
  using S = MfmaShape<FMT, NMAT, TR, RB, MR, NW>;
  constexpr bool CHAIN = S::CHAIN;
  // FP8: the item's 128-row scale blocks per matrix (its rows start on one)
  constexpr int FP8_NB = TR * MR > 128 ? TR * MR / 128 : 1;
  constexpr int D = S::D;
  static_assert(S::KSPLIT == KSPLIT, "shape");
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  // wave-uniform (readfirstlane: the compiler then keeps per-step branches scalar)
  const int rgrp = __builtin_amdgcn_readfirstlane(wave % RGRP);
  const int ksp = __builtin_amdgcn_readfirstlane(wave / RGRP);
  const int m16 = lane & 15, kg = lane >> 4;
  const size_t rb = row_bytes<FMT>(it.K);
  float *red = (float *)lds;  // k-split partials, after the last segment
  // An item is npass passes of TR rows (row0 + TR p ...).  The lane's row
  // group of pass p in the tiled layout (NULL past the matrix: loads read the
  // zero block).  K is a multiple of the k-step here, so rows are whole
  // 64-byte tiles: k-step s of the wave is tile column s, a 1 KB block of
  // which lane (m16, kg) reads piece kg of row m16.
  // (MR > 1: the item is MR passes, all in pass 0)
  const int npass = MR > 1 ? 1 : KSPLIT == 1 ? it.npass : 1;
  auto rows_of_pass = [&](const Item &x, int p, const uint8_t *(&ptr)[NMAT * MR]) {
#pragma unroll
    for (int rr = 0; rr < MR; rr++) {
      const int row = x.row0 + TR * (p * MR + rr) + rgrp * 16 + m16;
#pragma unroll
      for (int m = 0; m < NMAT; m++)
        ptr[m * MR + rr] =
            row < x.rows ? x.w[m] + (size_t)(row - m16) * rb + m16 * 64 + kg * 16 : nullptr;
    }
  };

  for (int g0 = 0; g0 < it.nroute; g0 += RG) {
    const int nr = min(RG, it.nroute - g0);
    // LDS holds the nr staged rows (rounded up to 4); columns per segment a
    // multiple of the k-steps the waves share
    const int rows_st = (nr + 3) & ~3;
    // MXFP4: the pass's e8m0 scales of the segment are staged too, NMAT x TR
    // rows of KS/32 bytes (+16: rows 80 B apart for KS 2048 fall in distinct
    // banks); segments are whole multiples of 512 columns, 16 scale bytes
    constexpr int SCB = FMT == FMT_MXFP4 ? NMAT * TR * MR : 0;  // scale rows of a pass
    constexpr int UNIT = FMT == FMT_MXFP4 && KSTEP * KSPLIT < 512 ? 512 : KSTEP * KSPLIT;
    // Whole K in one staged segment for every pass (the scales of all passes
    // staged with it) when it fits: the inputs are then staged once for all
    // passes.  Otherwise pass after pass, segment after segment.
    const int cap1 = (lds_bytes - rows_st * XPAD - SCB * npass * 16) /
                     (rows_st * 2 + (SCB * npass + 31) / 32);
    const bool one = cap1 >= it.K;
    const int KS = one ? it.K
                       : even_segment(it.K,
                                      (lds_bytes - rows_st * XPAD - SCB * 16) /
                                          (rows_st * 2 + (SCB + 31) / 32),
                                      UNIT);
    const int nseg = (it.K + KS - 1) / KS;
    const int STRIDE = KS * 2 + XPAD;
    const int SST = KS / 32 + 16;
    uint8_t *sc = lds + (size_t)rows_st * STRIDE;
    // B lanes past the routes read the last staged route: their output columns
    // are never stored (a column of the product depends on its B column only)
    int brow[RB];
#pragma unroll
    for (int nb = 0; nb < RB; nb++) brow[nb] = min(nb * 16 + m16, rows_st - 1);

    f32x4 acc[NMAT][MR][RB];
    for (int ps = 0; ps < npass * nseg; ps++) {
      const int p = ps / nseg, seg = ps - p * nseg;
      const int k0 = seg * KS;
      const bool last = seg == nseg - 1;
      if (seg == 0) {  // a pass's sums run over its segments
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
          for (int rr = 0; rr < MR; rr++)
#pragma unroll
            for (int nb = 0; nb < RB; nb++) acc[m][rr][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const uint8_t *cur[NMAT * MR];
      rows_of_pass(it, p, cur);
      // chained: the rows the last segment's last iterations load from -- the
      // next pass's, the next route group's first pass's, the next item's,
      // or none
      const uint8_t *succ[NMAT * MR];
#pragma unroll
      for (int q = 0; q < NMAT * MR; q++) succ[q] = nullptr;
      if (CHAIN && last) {
        if (p + 1 < npass) {
          rows_of_pass(it, p + 1, succ);
        } else if (g0 + RG < it.nroute) {
          rows_of_pass(it, 0, succ);
        } else if (S::XCHAIN && has_nxt) {
          rows_of_pass(nxt, 0, succ);
        }
      }
      const int kn = min(KS, it.K - k0);
      const int nsteps = kn / KSTEP;  // k-steps of this segment (chained: a multiple of D)
      const int my_steps = (nsteps - ksp + KSPLIT - 1) / KSPLIT;  // s = ksp + KSPLIT * i

      auto load = [&](u32x4(&r)[NMAT * MR], int i) {
        const int s = ksp + KSPLIT * i;
        const int c0 = k0 + s * KSTEP;
        const bool past = CHAIN && c0 >= it.K;  // the successor's k-step c0 - K
        const int ts = (past ? c0 - it.K : c0) / KSTEP;  // tile column of the k-step
#pragma unroll
        for (int q = 0; q < NMAT * MR; q++) {
          // non-temporal: the wave reads whole 1 KB tiles, so no line is
          // wanted again, and the staged input rows keep their place in L2
          const uint8_t *base = past ? succ[q] : cur[q];
          const bool ok = (CHAIN || i < my_steps) && base != nullptr;
          r[q] = gload16_nt(ok ? (const void *)(base + (size_t)ts * 1024) : zero16());
        }
      };

      // chained: a later segment's, pass's, route group's or (pre) item's
      // first k-steps were loaded by the iterations before it
      if (!CHAIN || (ps == 0 && g0 == 0 && !pre)) {
#pragma unroll
        for (int d = 0; d < D; d++) load(raw[d], d);
      }

      if (ps == 0 || !one) {
        // gate+up: a later segment's loads are issued before the barrier that
        // frees the LDS of the previous one
        constexpr bool EARLY = NMAT == 2;
        if (!EARLY || k0 == 0) {  // the route group's rows (and an FP8 pass's block scales)
          __syncthreads();  // previous readers of the LDS are done
          if (k0 == 0 && (g0 == 0 || !one))
            stage_scales<FMT, NMAT, (FMT == FMT_FP8 ? FP8_NB : 1), NT>(s_lds, it,
                                                                                  it.row0 + TR * p);
          route_rows<RG>(rows_lds, it, g0, nr);
          __syncthreads();
        }
        stage_segment<FMT, NMAT, TR, MFMA_SB, EARLY, NT>(lds, sc, SST, it, rows_lds, nr, k0, kn,
                                                     STRIDE, k0 > 0, one ? 0 : p * MR,
                                                     one ? npass * MR : MR);
        __syncthreads();
      }
      // this pass's staged scale rows
      const uint8_t *scp = sc + (size_t)(one ? p * SCB : 0) * SST;

      for (int i0 = 0; i0 < my_steps; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
          const int i = i0 + d;
          {  // steps past my_steps run too: zero A (from the zero block), and
             // B and scale reads kept inside the segment
            const int s = ksp + KSPLIT * (i < my_steps ? i : my_steps - 1);
            const int lcol = s * KSTEP + kg * EPC;  // column within the segment
            f32x4 part[NMAT][MR][RB];
            if constexpr (FMT == FMT_FP8) {
#pragma unroll
              for (int m = 0; m < NMAT; m++)
#pragma unroll
                for (int rr = 0; rr < MR; rr++)
#pragma unroll
                  for (int nb = 0; nb < RB; nb++) part[m][rr][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if constexpr (MR > 1) {
              // several row groups: each eighth of a chunk is decoded just
              // before its MFMAs, and each B chunk from the LDS serves both
              // matrices and the MR row groups (the sums run in the same order
              // as below)
              float scl[NMAT][MR];
#pragma unroll
              for (int m = 0; m < NMAT; m++)
#pragma unroll
                for (int rr = 0; rr < MR; rr++)
                  scl[m][rr] = FMT == FMT_MXFP4
                                   ? e8m0_to_f32(scp[(size_t)(rr * NMAT * TR + m * TR + rgrp * 16 +
                                                              m16) * SST + (lcol >> 5)])
                                   : 1.0f;
              static_for<JM>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                u32x4 b[RB];
#pragma unroll
                for (int nb = 0; nb < RB; nb++)
                  b[nb] = *(const u32x4 *)(lds + (size_t)brow[nb] * STRIDE + (size_t)(lcol + 8 * j) * 2);
#pragma unroll
                for (int rr = 0; rr < MR; rr++)
#pragma unroll
                  for (int m = 0; m < NMAT; m++) {
                    const u32x4 a = decode_part<FMT, j>(raw[d][m * MR + rr], scl[m][rr]);
#pragma unroll
                    for (int nb = 0; nb < RB; nb++) {
                      if constexpr (FMT == FMT_FP8)
                        part[m][rr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b[nb]),
                            part[m][rr][nb], 0, 0, 0);
                      else
                        acc[m][rr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b[nb]),
                            acc[m][rr][nb], 0, 0, 0);
                    }
                  }
              });
            } else {
            Dec<FMT> dec[NMAT][MR];
#pragma unroll
            for (int m = 0; m < NMAT; m++)
#pragma unroll
              for (int rr = 0; rr < MR; rr++) {
                if constexpr (FMT == FMT_MXFP4)
                  decode_scaled_fp4(
                      raw[d][m * MR + rr],
                      e8m0_to_f32(scp[(size_t)(rr * NMAT * TR + m * TR + rgrp * 16 + m16) * SST +
                                      (lcol >> 5)]),
                      dec[m][rr]);
                else
                  decode<FMT>(raw[d][m * MR + rr], dec[m][rr]);
              }
            // each B chunk from the LDS serves both matrices and the MR row groups
#pragma unroll
            for (int j = 0; j < JM; j++) {
#pragma unroll
              for (int nb = 0; nb < RB; nb++) {
                const u32x4 b = *(const u32x4 *)(lds + (size_t)brow[nb] * STRIDE +
                                                 (size_t)(lcol + 8 * j) * 2);
#pragma unroll
                for (int rr = 0; rr < MR; rr++)
#pragma unroll
                  for (int m = 0; m < NMAT; m++) {
                    const u32x4 a = {dec[m][rr].v[4 * j], dec[m][rr].v[4 * j + 1],
                                     dec[m][rr].v[4 * j + 2], dec[m][rr].v[4 * j + 3]};
                    if constexpr (FMT == FMT_FP8)
                      part[m][rr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                          __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                          part[m][rr][nb], 0, 0, 0);
                    else
                      acc[m][rr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                          __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                          acc[m][rr][nb], 0, 0, 0);
                  }
              }
            }
            }
            if constexpr (FMT == FMT_FP8) {
              // a k-step's 64 columns sit in one 128-column scale block; row
              // group rr of matrix m in the item's 128-row block (TR rr) / 128,
              // slot m FP8_NB + that block
              static_assert(NMAT * FP8_NB <= 4, "scale slots");
#pragma unroll
              for (int m = 0; m < NMAT; m++)
#pragma unroll
                for (int rr = 0; rr < MR; rr++) {
                  const float sc8 =
                      s_lds[(m * FP8_NB + ((TR * rr) >> 7)) * 128 + ((k0 + s * KSTEP) >> 7)];
#pragma unroll
                  for (int nb = 0; nb < RB; nb++) acc[m][rr][nb] += part[m][rr][nb] * sc8;
                }
            }
            load(raw[d], i + D);
          }
        }
      }
      if (!last) continue;  // the pass goes on in its next segment
      // sum the k-splits: waves with ksp > 0 park their partials in LDS
      if constexpr (KSPLIT > 1) {
        __syncthreads();
        if (ksp > 0) {
#pragma unroll
          for (int m = 0; m < NMAT; m++)
            *(f32x4 *)(red + (((size_t)(ksp - 1) * RGRP + rgrp) * NMAT + m) * 256 + lane * 4) =
                acc[m][0][0];
        }
        __syncthreads();
        if (ksp == 0) {
          for (int kk = 1; kk < KSPLIT; kk++)
#pragma unroll
            for (int m = 0; m < NMAT; m++)
              acc[m][0][0] +=
                  *(const f32x4 *)(red + (((size_t)(kk - 1) * RGRP + rgrp) * NMAT + m) * 256 +
                                   lane * 4);
        }
      }
      if (ksp == 0) {
        // lane holds rows 4*kg + t (t < 4) of its row group, for route nb*16 + m16
#pragma unroll
        for (int rr = 0; rr < MR; rr++)
#pragma unroll
        for (int nb = 0; nb < RB; nb++) {
          if (nb * 16 + m16 >= nr) continue;
          const int orow0 = it.row0 + TR * (p * MR + rr) + rgrp * 16 + 4 * kg;
          const size_t o = (size_t)rows_lds[ROWS_OUT + nb * 16 + m16] * it.rows + orow0;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; t++) {
            v[t] = acc[0][rr][nb][t];
            if constexpr (NMAT == 2) v[t] = v[t] * sigmoidf_(v[t]) * acc[1][rr][nb][t];
          }
          if constexpr (NMAT == 2) {  // 4 consecutive bf16 act values (rows % 16 == 0)
            if (orow0 < it.rows) {
              u32x2 pk;
              pk.x = pack_bf16x2(v[0], v[1]);
              pk.y = pack_bf16x2(v[2], v[3]);
              *(u32x2 *)((uint16_t *)it.out + o) = pk;
            }
          } else {
#pragma unroll
            for (int t = 0; t < 4; t++)
              if (orow0 + t < it.rows) ((float *)it.out)[o + t] = v[t];
          }
        }
      }
    }
  }
  return S::XCHAIN && has_nxt;
}

// ------------------------------------------------------------------ one-row down + blend

// A step of one token row, where the down pass streams few bytes and its
// time is latency: the down GEMV and the blend in one kernel.  Workgroup b
// owns output columns [4 b, 4 b + 4) -- those rows of every down matrix --
// for all of the row's sources: its k slots (k <= 32) and the shared expert.
// A wave takes one source at a time; lane l = 16 p + 4 i + q holds row
// 4 b + i, piece q of tile column j and K part p = j % 4, so every
// (column, source) sum is built as the down pass's VALU path builds it: each
// lane sums its chunks of part p in ascending j, quad_sum over q, then the
// parts in order ((p0 + p1) + p2) + p3.  y and the output are therefore
// bitwise those of the down pass and blend_kernel.  Then the output columns
// are blended in slot order and the shared expert last, in fp32 with one
// rounding.  Nothing crosses workgroups.
constexpr int DB1_ROWS = 4;  // output columns per workgroup

template <int FMT>
__global__ __launch_bounds__(EX_THREADS) void down_blend1_kernel(Down1Args a) {
  constexpr int EPC = ChunkElems<FMT>::value;
  constexpr int LB = Lds<FMT>::bytes;  // act element: bf16, fp32 for fp32 experts
  constexpr int D = 4;                 // tile columns of loads in flight per lane
  constexpr int MAXS = 33;             // k <= 32 slots and the shared expert
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // act rows, then y
  __shared__ const uint8_t *s_w[MAXS];
  __shared__ const void *s_s[MAXS];
  __shared__ int s_p[MAXS];
  __shared__ int s_z[MAXS];  // a zero-computation expert's slot: adds w * x
  const int tid = threadIdx.x;
  const int wave = tid / WAVE, lane = tid % WAVE;
  const int p = lane >> 4, ri = (lane >> 2) & 3, q = lane & 3;
  const int k = a.k, NS = k + (a.sh_w ? 1 : 0);
  const int K = a.K;  // routed and shared K are equal on this path
  const int row0 = blockIdx.x * DB1_ROWS;
  const int rows = min(DB1_ROWS, a.h - row0);
  const int row = row0 + ri;
  const bool row_ok = ri < rows;
  const size_t rb = row_bytes<FMT>(K);
  const int STR = K * LB + XPAD;  // staged act row stride
  float *ylds = (float *)(lds + (size_t)NS * STR);  // [DB1_ROWS][NS]

  // the sources: weight and scale matrices, act position (-1: dropped slot)
  if (tid < NS) {
    if (tid < k) {
      const int pos = a.route_pos[tid];
      const int e = a.idx[tid];
      s_p[tid] = pos;
      s_z[tid] = e >= a.E && e < a.E + a.Z;
      s_w[tid] = pos >= 0 ? (const uint8_t *)a.w[e] : nullptr;
      s_s[tid] = pos >= 0 && a.s ? a.s[e] : nullptr;
    } else {
      s_p[tid] = 0;
      s_z[tid] = 0;
      s_w[tid] = (const uint8_t *)a.sh_w;
      s_s[tid] = a.sh_s;
    }
  }
  __syncthreads();

  // this wave's units: sources j = wave + 4 u; steps i of a unit: tile column
  // p + 4 i of the lane's part; the load stream runs D steps ahead, on from
  // one unit into the next
  const int cn = K / EPC;
  const int nj = (cn + 3) >> 2;         // tile columns
  const int nsu = (nj + VPARTS - 1) / VPARTS;  // steps per unit
  const int nu = NS > wave ? (NS - wave + 3) / 4 : 0;
  const int T = nu * nsu;
  struct Ld {
    u32x4 raw;
    uint32_t sb;  // MXFP4 scale byte
    float sc;     // FP8 block scale
  };
  auto load = [&](Ld &b, int t) {
    b.raw = u32x4{0, 0, 0, 0};
    b.sb = 127;
    b.sc = 1.f;
    const int uu = t / nsu, st = t - uu * nsu;
    const int j = wave + 4 * uu;
    const int c = 4 * (p + VPARTS * st) + q;
    if (t < T && c < cn && row_ok) {
      const uint8_t *wm = s_w[j];
      if (wm) {
        b.raw = __builtin_nontemporal_load((const u32x4 *)(wm + tile_off(row, c, rb)));
        if constexpr (FMT == FMT_MXFP4)
          b.sb = ((const uint8_t *)s_s[j])[(size_t)row * (K >> 5) + c];
        if constexpr (FMT == FMT_FP8)
          b.sc = ((const float *)s_s[j])[(size_t)(row >> 7) * ((K + 127) >> 7) + ((c * EPC) >> 7)];
      }
    }
  };
  Ld buf[D];
#pragma unroll
  for (int d = 0; d < D; d++) load(buf[d], d);  // in flight during the staging below

  // stage the act rows (zeros for dropped slots), 8 loads per thread per trip
  {
    const int q16 = K * LB / 16;  // 16-byte pieces per row
    const int total = NS * q16;
    for (int i0 = tid; i0 < total; i0 += 8 * EX_THREADS) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int i = i0 + u * EX_THREADS;
        v[u] = u32x4{0, 0, 0, 0};
        if (i < total) {
          const int j = i / q16, qq = i - j * q16;
          const int pos = s_p[j];
          if (pos >= 0)
            v[u] = j < k ? ((const u32x4 *)((const uint8_t *)a.act + (size_t)pos * K * LB))[qq]
                         : ((const u32x4 *)a.act_sh)[qq];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int i = i0 + u * EX_THREADS;
        if (i < total) {
          const int j = i / q16, qq = i - j * q16;
          *(u32x4 *)(lds + (size_t)j * STR + (size_t)qq * 16) = v[u];
        }
      }
    }
  }
  __syncthreads();

  float acc = 0.f;
  for (int s0 = 0; s0 < T; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      const int t = s0 + d;
      if (t < T) {
        const int uu = t / nsu, st = t - uu * nsu;
        const int j = wave + 4 * uu;
        const int c = 4 * (p + VPARTS * st) + q;
        if (c < cn) {
          uint32_t xr[Dec<FMT>::WORDS];
          const uint8_t *xl = lds + (size_t)j * STR + (size_t)c * EPC * LB;
#pragma unroll
          for (int w4 = 0; w4 < Dec<FMT>::WORDS; w4 += 4) {
            const u32x4 xv = *(const u32x4 *)(xl + 4 * w4);
            xr[w4] = xv.x;
            xr[w4 + 1] = xv.y;
            xr[w4 + 2] = xv.z;
            xr[w4 + 3] = xv.w;
          }
          Dec<FMT> dec;
          decode<FMT>(buf[d].raw, dec);
          if constexpr (FMT == FMT_FP8 || FMT == FMT_MXFP4) {
            const float sc = FMT == FMT_FP8 ? buf[d].sc : e8m0_to_f32(buf[d].sb);
            acc = fmaf(chunk_dot_regs<FMT>(dec, xr, 0.f), sc, acc);
          } else {
            acc = chunk_dot_regs<FMT>(dec, xr, acc);
          }
        }
        load(buf[d], t + D);
        if (st == nsu - 1) {  // unit complete: lane sums, the parts in order
          const float v = quad_sum(acc);
          const float v1 = __shfl(v, lane + 16, WAVE);
          const float v2 = __shfl(v, lane + 32, WAVE);
          const float v3 = __shfl(v, lane + 48, WAVE);
          if (p == 0 && q == 0 && row_ok) ylds[ri * NS + j] = ((v + v1) + v2) + v3;
          acc = 0.f;
        }
      }
    }
  }
  __syncthreads();

  // blend: slot order, then the shared expert (a dropped slot adds nothing,
  // a zero expert's slot the input column)
  if (tid < rows) {
    float o = 0.f;
    float xc = 0.f;
    if (a.Z > 0) {
      if constexpr (FMT == FMT_F32)
        xc = ((const float *)a.x)[row0 + tid];
      else
        xc = __uint_as_float((uint32_t)((const uint16_t *)a.x)[row0 + tid] << 16);
    }
    for (int j = 0; j < k; j++) {
      if (s_p[j] >= 0) o = fmaf(a.w_slot[j], ylds[tid * NS + j], o);
      else if (s_z[j]) o = fmaf(a.w_slot[j], xc, o);
    }
    if (a.sh_w) o = fmaf(a.g ? a.g[0] : 1.f, ylds[tid * NS + k], o);
    if constexpr (FMT == FMT_F32)
      ((float *)a.out)[row0 + tid] = o;
    else
      ((uint16_t *)a.out)[row0 + tid] = (uint16_t)f32_to_bf16_bits(o);
  }
}

// Kernel modes.  MODE_MIXED: items of two or more routes go down the MFMA
// path, single-route ones down the VALU path (a step where experts can have
// more than 4 routes).  MODE 1, 2, 4: VALU path only, route groups of up to
// MODE (the most routes an expert can have in the step).  Each kernel holds
// only its own paths: unexecuted code still costs registers and instruction
// cache lines.
constexpr int MODE_MIXED = 0;
// MODE_GEMM: steps whose experts average 32 or more routes (large N), the
// grouped-GEMM form: every item takes route groups of 64 (four 16-route MFMA
// blocks per decoded weight fragment), a single route too.  Workgroups of 8
// waves, one a CU, on 128-row tiles: an item is MR of them (256 gate+up or
// 512 down rows), so each staged input segment feeds 256 or 512 rows, and
// the LDS of the whole CU holds segments of 1024 columns.  (4-wave
// workgroups, two a CU, on items of half the rows measured 4-7 % slower.)
constexpr int MODE_GEMM = 8;
constexpr int GEMM_WAVES = 8;
constexpr int GEMM_TR = 128;
constexpr int GEMM_RB = 4;
static_assert(16 * GEMM_RB == SH_CHUNK_GEMM, "shared-expert chunks are route groups");

// One pass over the items (see the kernel modes above).
// Workgroups per CU the kernel is built for: beside the MFMA path as
// mixed_blocks_per_cu says, one of 8 waves in the grouped-GEMM form, 2 of 4
// waves elsewhere (measured on MI355X).
template <int NMAT, int MODE>
constexpr int kMinBlocks =
    MODE == MODE_MIXED ? mixed_blocks_per_cu(NMAT) : MODE == MODE_GEMM ? 1 : 2;
template <int MODE>
constexpr int kThreads = MODE == MODE_GEMM ? GEMM_WAVES * WAVE : EX_THREADS;

// Item `item` of a pass: the shared expert's tiles first, then the tiles of
// the active experts, tile-fastest.  The first `big` routed items cover npass
// tiles each; past them the last tail experts' items cover one tile each
// (big = INT_MAX: none such).  The slot is clamped into the compaction
// arrays and the expert id into [0, E), so a workgroup may read its first
// item before it knows how many items there are (no-ops for a real item).
template <int NMAT, int TR>
__device__ __forceinline__ Item make_item(const GemvArgs &a, int item, int big = INT_MAX) {
  Item it;
  int tile;
  if (item < a.sh_items) {  // tile-fastest over the chunks of the N routes
    it.w[0] = (const uint8_t *)a.sh_w0;
    it.s[0] = a.sh_s0;
    it.w[1] = (const uint8_t *)a.sh_w1;
    it.s[1] = a.sh_s1;
    const int chunk = item / a.sh_tiles;
    tile = item - chunk * a.sh_tiles;
    it.rows = a.sh_rows;
    it.K = a.sh_K;
    it.route_base = chunk * a.sh_chunk;
    it.nroute = min(a.sh_chunk, a.N - it.route_base);
    it.route_map = nullptr;
    it.out_map = nullptr;
    it.src = a.sh_src;
    it.out = a.sh_out;
  } else {
    // `big` items of npass tiles, then the tail experts' one-tile items
    int q = item - a.sh_items, s0 = 0, per = a.tiles;
    it.npass = a.npass;
    if (q >= big) {
      s0 = big / a.tiles;
      q -= big;
      per = (a.rows + TR - 1) / TR;
      it.npass = 1;
    }
    const int qs = q / per;
    const int slot = min(s0 + qs, a.max_active - 1);
    const int e = min(max(a.active[slot], 0), a.E - 1);
    tile = q - qs * per;
    it.w[0] = (const uint8_t *)a.w0[e];
    it.s[0] = a.s0 ? a.s0[e] : nullptr;
    it.w[1] = NMAT == 2 ? (const uint8_t *)a.w1[e] : nullptr;
    it.s[1] = (NMAT == 2 && a.s1) ? a.s1[e] : nullptr;
    it.rows = a.rows;
    it.K = a.K;
    it.route_base = a.off[slot];
    it.nroute = a.off[slot + 1] - it.route_base;
    it.route_map = a.src_by_token ? a.route_tok : nullptr;
    it.out_map = a.out_map;
    it.src = a.src;
    it.out = a.out;
  }
  if (item < a.sh_items) it.npass = a.sh_npass;
  it.row0 = tile * TR * it.npass;
  return it;
}

template <int FMT, int NMAT, int TR, int MODE>
__global__ __launch_bounds__((kThreads<MODE>), (kMinBlocks<NMAT, MODE>)) void expert_kernel(GemvArgs a) {
  // inputs: bf16 x rows or bf16 act rows, fp32 for fp32 experts
  constexpr bool SRC_F32 = FMT == FMT_F32;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // a.lds_bytes
  __shared__ float s_lds[(MODE == MODE_GEMM ? 4 : 2) * 128];  // FP8 block-scale slots
  __shared__ int rows_lds[2 * ROWS_OUT];
  __shared__ float vred[VPARTS * 16 * 2 * 4];  // VALU 16-row items: the K parts' sums
  // decode steps (VALU path only): the first item's descriptor is read
  // beside the item count, so its weight loads wait for two dependent round
  // trips rather than three.  Beside the MFMA path the kernels measured
  // slower with it (FP8 gate+up, MXFP4 down), so they read it after.
  constexpr bool SPEC = MODE != MODE_MIXED && MODE != MODE_GEMM;
  Item first;
  if constexpr (SPEC) first = make_item<NMAT, TR>(a, blockIdx.x);
  const int n_active = min(*a.n_active, a.max_active);
  // the last tail_e experts in one-tile items, so that the pass ends on
  // short items (tail_e is 0 in the VALU modes, where the first item is read
  // before the count)
  const int n_tail = min(n_active, a.tail_e);
  const int big = (n_active - n_tail) * a.tiles;
  const int n_items = a.sh_items + big + n_tail * ((a.rows + TR - 1) / TR);
  if constexpr (!SPEC) {
    if (blockIdx.x < n_items) first = make_item<NMAT, TR>(a, blockIdx.x, big);
  }
  if constexpr (MODE == MODE_GEMM || MODE == MODE_MIXED) {
    // the host launches these modes only where every K suits the MFMA path
    static_assert(FMT != FMT_F32 && TR >= 16, "no MFMA path for this shape");
    static_assert(MODE != MODE_GEMM || TR == GEMM_TR, "no grouped-GEMM path for this shape");
    constexpr bool G = MODE == MODE_GEMM;
    constexpr int RB = G ? GEMM_RB : 1;
    constexpr int MR = G ? gemm_mr(FMT, NMAT) : 1;
    constexpr int NW = G ? GEMM_WAVES : EX_WAVES;
    using S = MfmaShape<FMT, NMAT, TR, RB, MR, NW>;
    u32x4 ring[S::D][NMAT * MR];  // the MFMA path's k-steps in flight
    bool pre = false;        // ring holds the item's first k-steps
    Item it = first;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
      const int ni = item + gridDim.x;
      if constexpr (!S::XCHAIN) {
        if (item != blockIdx.x) it = make_item<NMAT, TR>(a, item, big);
      }
      // chained shapes: the next item, read now; if it is an MFMA item of the
      // same K, this item's last iterations load its first k-steps
      Item nx;
      bool chain = false;
      if constexpr (S::XCHAIN) {
        if (ni < n_items) {
          nx = make_item<NMAT, TR>(a, ni, big);
          chain = nx.nroute > 1 && nx.K == it.K;
        }
      }
      // (grouped-GEMM items: a single route too goes down the MFMA path,
      // whose B lanes past the routes are never stored)
      if (G || it.nroute > 1) {
        pre = mfma_item<FMT, NMAT, TR, SRC_F32, RB, MR, NW>(lds, a.lds_bytes, s_lds, rows_lds, it,
                                                            ring, pre, nx, chain);
      } else if constexpr (!G) {
        for (int p = 0; p < it.npass; p++) {  // the item's passes of TR rows
          Item sub = it;
          sub.row0 = it.row0 + TR * p;
          valu_item<FMT, NMAT, TR, SRC_F32, 1>(lds, a.lds_bytes, s_lds, rows_lds, vred, sub);
        }
        pre = false;
      }
      if constexpr (S::XCHAIN) {
        if (ni < n_items) it = nx;
      }
    }
  } else {
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
      const Item it = item == blockIdx.x ? first : make_item<NMAT, TR>(a, item, big);
      if (MODE == 1 || it.nroute <= 1)
        valu_item<FMT, NMAT, TR, SRC_F32, 1>(lds, a.lds_bytes, s_lds, rows_lds, vred, it);
      else if (MODE == 2 || it.nroute <= 2)
        valu_item<FMT, NMAT, TR, SRC_F32, 2>(lds, a.lds_bytes, s_lds, rows_lds, vred, it);
      else
        valu_item<FMT, NMAT, TR, SRC_F32, 4>(lds, a.lds_bytes, s_lds, rows_lds, vred, it);
    }
  }
}

template <int FMT, int NMAT, int TR>
hipError_t go(bool mfma, const GemvArgs &a, int grid, hipStream_t s, hipEvent_t e0,
              hipEvent_t e1) {
  if constexpr (FMT != FMT_F32 && TR == 64) {
    if (mfma && a.gemm) {  // experts average 32 or more routes
      hipExtLaunchKernelGGL((expert_kernel<FMT, NMAT, GEMM_TR, MODE_GEMM>), dim3(grid),
                            dim3(kThreads<MODE_GEMM>), a.lds_bytes, s, e0, e1, 0, a);
      return hipGetLastError();
    }
  }
  if constexpr (FMT != FMT_F32) {
    if (mfma) {  // some expert may have more than 4 routes
      hipExtLaunchKernelGGL((expert_kernel<FMT, NMAT, TR, MODE_MIXED>), dim3(grid),
                            dim3(EX_THREADS), a.lds_bytes, s, e0, e1, 0, a);
      return hipGetLastError();
    }
  }
  if (a.max_r <= 1)
    hipExtLaunchKernelGGL((expert_kernel<FMT, NMAT, TR, 1>), dim3(grid), dim3(EX_THREADS),
                          a.lds_bytes, s, e0, e1, 0, a);
  else if (a.max_r <= 2)
    hipExtLaunchKernelGGL((expert_kernel<FMT, NMAT, TR, 2>), dim3(grid), dim3(EX_THREADS),
                          a.lds_bytes, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL((expert_kernel<FMT, NMAT, TR, 4>), dim3(grid), dim3(EX_THREADS),
                          a.lds_bytes, s, e0, e1, 0, a);
  return hipGetLastError();
}

template <int FMT, int NMAT>
hipError_t go_shape(bool mfma, int tr, const GemvArgs &a, int grid, hipStream_t s,
                    hipEvent_t e0, hipEvent_t e1) {
  if (tr == 16) return go<FMT, NMAT, 16>(mfma, a, grid, s, e0, e1);
  return go<FMT, NMAT, 64>(mfma, a, grid, s, e0, e1);
}

}  // namespace

// one weight format's one-row down + blend (experts_<fmt>.hip)
template <int FMT>
hipError_t launch_down_blend1_fmt(const Down1Args &a, int lds_bytes, hipStream_t s, hipEvent_t e0,
                                  hipEvent_t e1) {
  const dim3 grid((a.h + DB1_ROWS - 1) / DB1_ROWS), block(EX_THREADS);
  hipExtLaunchKernelGGL((down_blend1_kernel<FMT>), grid, block, lds_bytes, s, e0, e1, 0, a);
  return hipGetLastError();
}

// one weight format's kernels (experts_<fmt>.hip)
template <int FMT>
hipError_t launch_expert_fmt(bool mfma, int nmat, int tr, const GemvArgs &a, int grid,
                             hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return nmat == 2 ? go_shape<FMT, 2>(mfma, tr, a, grid, s, e0, e1)
                   : go_shape<FMT, 1>(mfma, tr, a, grid, s, e0, e1);
}

}  // namespace moe
