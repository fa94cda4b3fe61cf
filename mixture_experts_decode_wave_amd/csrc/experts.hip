// Dispatch of the expert passes to the per-format kernel files, and the
// host-side choice of their launch shape.
#include <atomic>

#include "device.h"
#include "launch.h"

namespace moe {

hipError_t launch_expert_f32(bool, int, int, const GemvArgs &, int, hipStream_t, hipEvent_t,
                             hipEvent_t);
hipError_t launch_expert_bf16(bool, int, int, const GemvArgs &, int, hipStream_t, hipEvent_t,
                              hipEvent_t);
hipError_t launch_expert_fp8(bool, int, int, const GemvArgs &, int, hipStream_t, hipEvent_t,
                             hipEvent_t);
hipError_t launch_expert_mxfp4(bool, int, int, const GemvArgs &, int, hipStream_t, hipEvent_t,
                               hipEvent_t);
hipError_t launch_down_blend1_f32(const Down1Args &, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_down_blend1_bf16(const Down1Args &, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_down_blend1_fp8(const Down1Args &, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_down_blend1_mxfp4(const Down1Args &, int, hipStream_t, hipEvent_t, hipEvent_t);

constexpr long MAX_LDS = 65536;  // dynamic LDS of an expert pass at most
// and of its grouped-GEMM form, one workgroup a CU: 64 routes x 1024 columns
// of bf16 inputs and 512 MXFP4 scale rows of them (153 KB), with the kernel's
// static LDS within the CU's 160 KB
constexpr long GEMM_LDS = 157696;

// Largest tile (64 or 16 weight rows) that still gives >= min_items items at
// the most active experts; smaller tiles keep a decode step of a few experts
// spread over all 256 CUs.
int expert_tile_rows(int K, int rows, int max_active, int min_items) {
  (void)K;
  if ((long)max_active * ((rows + 63) / 64) >= min_items) return 64;
  return 16;
}

// Dynamic LDS of a launch: room for the VALU path's largest route group (4)
// and the MFMA path's 16 routes at their smallest segment (plus its k-split
// partials), and beyond that for the whole K of the largest route group the
// step can have, up to 64 KB, so decode steps keep their LDS small and their
// occupancy high.
static int expert_lds_bytes(bool with_mfma, bool gemm, int fmt, int nmat, int tr, int K,
                            int max_r) {
  const int epc = fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 8 : fmt == FMT_FP8 ? 16 : 32;
  const int lb = fmt == FMT_F32 ? 4 : 2;
  const int pad = 16;
  int need = 4 * (4 * epc * lb + pad);  // the VALU path's 4 routes, one tile column
  int rg = max_r <= 1 ? 1 : max_r <= 2 ? 2 : 4;
  if (with_mfma) {
    const int ksplit = 64 / tr;
    int m = 16 * (4 * epc * ksplit * 2 + pad);
    if (fmt == FMT_MXFP4)  // 512-column segments with the tile's staged scales
      m = 16 * (512 * 2 + pad) + nmat * tr * (512 / 32 + 16);
    if (m > need) need = m;
    const int red = (ksplit - 1) * (tr / 16) * nmat * 1024;  // 16x16 fp32 partials
    if (red > need) need = red;
    rg = max_r >= 16 ? 16 : (max_r + 3) & ~3;  // MFMA route groups, staged in 4s
    if (gemm) {  // route groups of 64, the smallest segment of each
      rg = 64;
      m = fmt == FMT_MXFP4 ? 64 * (512 * 2 + pad) + nmat * tr * gemm_mr(fmt, nmat) * (512 / 32 + 16)
                           : 64 * (4 * epc * 2 + pad);
      if (m > need) need = m;
    }
  }
  long want = (long)rg * ((long)K * lb + pad);
  // the down pass beside the MFMA path runs 3 workgroups per CU: 48 KB each;
  // the grouped-GEMM form one per CU, with the CU's whole LDS: its longest
  // segments
  const long cap = gemm ? GEMM_LDS : with_mfma && nmat == 1 ? 49152 : MAX_LDS;
  if (gemm) want = cap;
  if (want > cap) want = cap;
  if (want > need) need = (int)want;
  return (need + 15) & ~15;
}

static hipError_t launch_fmt(bool mfma, int fmt, int nmat, int tr, const GemvArgs &a, int grid,
                             hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (fmt) {
    case FMT_F32: return launch_expert_f32(mfma, nmat, tr, a, grid, s, e0, e1);
    case FMT_BF16: return launch_expert_bf16(mfma, nmat, tr, a, grid, s, e0, e1);
    case FMT_FP8: return launch_expert_fp8(mfma, nmat, tr, a, grid, s, e0, e1);
    default: return launch_expert_mxfp4(mfma, nmat, tr, a, grid, s, e0, e1);
  }
}

// Compute units of the current device (cached per device; 0 if unknown).
static int cu_count() {
  static std::atomic<int> cus[64];
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 0;
  int n = cus[d].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) n = 0;
    cus[d].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_expert_gemv(int fmt, int nmat, const GemvArgs &a0, int max_items, int tr,
                              int max_r, bool wide, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  const int cap = 256 * 8;
  const int K = a0.K > a0.sh_K ? a0.K : a0.sh_K;
  // the MFMA path once experts can have more than 4 routes (more than 4 rows);
  // up to that the VALU path's route groups of 2 and 4 serve best.  Its k-steps
  // take 4 chunks of every row: K must be a multiple of that.
  // (MXFP4: multiples of 512, so staged scale rows move in 16-byte pieces)
  const int kstep = fmt == FMT_MXFP4 ? 512 : 4 * (fmt == FMT_BF16 ? 8 : 16);
  const bool with_mfma = fmt != FMT_F32 && tr >= 16 && max_r > 4 && a0.K % kstep == 0 &&
                         (a0.sh_w0 == nullptr || a0.sh_K % kstep == 0);
  GemvArgs a = a0;
  a.gemm = with_mfma && wide && tr == 64;
  const int t8 = a.gemm ? 2 : 1;  // 64-row tiles of a kernel tile (the grouped-GEMM form's: 128 rows)
  // Beside the MFMA path an item of a routed expert may span npass 64-row
  // tiles: its inputs are staged once for all of them when they fit the LDS
  // in one segment, and its weight loads run on from tile to tile.  As many
  // (up to 4, FP8 2: an item stays in one 128-row scale block) as keep
  // >= 2048 items, 8 per CU.
  int npass = 1;
  const int tiles0 = a0.tiles;
  const long experts = tiles0 > 0 ? max_items / tiles0 : 0;
  if (a.gemm) {
    npass = gemm_mr(fmt, nmat);  // computed together, not pass after pass
  } else if (with_mfma && tr == 64) {
    const int most = fmt == FMT_FP8 ? 2 : 4;
    while (npass < most && experts * ((tiles0 + 2 * npass - 1) / (2 * npass)) >= 2048) npass *= 2;
  }
  a.tiles = (tiles0 + t8 * npass - 1) / (t8 * npass);
  a.npass = npass;
  // Beside the MFMA path the gate+up pass's last experts take one-tile
  // items, about one for each resident workgroup: the pass then ends on short
  // items (DeepSeek-V3-shaped layer, 64 rows: gate+up 697 -> 690 us; in the
  // down pass, with its shorter items, it measured as often slower as faster)
  a.tail_e = 0;
  if (with_mfma && !a.gemm && nmat == 2 && npass > 1 && tiles0 > 0) {
    const int slots = mixed_blocks_per_cu(nmat) * cu_count();
    a.tail_e = (slots + tiles0 - 1) / tiles0;
  }
  {
    const long tail = experts < a.tail_e ? experts : a.tail_e;
    max_items = (int)((experts - tail) * a.tiles + tail * tiles0);
  }
  // beside the MFMA path the shared expert's N routes come in chunks of one
  // route group, each chunk an item of its own: its tiles then spread over
  // workgroups, where one workgroup walking every route group of a tile was
  // the pass's tail (MXFP4 verify layer at 256 rows: gate+up 454 us against
  // 404 us without the shared expert; chunked, 432 us; at 1024 rows
  // 954 -> 694 us).  The down pass chunks too, one tile an item: its shared
  // items walking all N routes were the pass's longest (at 256 rows 235 ->
  // 232 us; no change at 64 rows, where the chunks are 4)
  const bool chunk = with_mfma;
  a.sh_chunk = chunk ? (a.gemm ? SH_CHUNK_GEMM : SH_CHUNK_MIXED) : (a0.N > 0 ? a0.N : 1);
  // the down pass's shared items stay one tile each (its items are short)
  a.sh_npass = chunk && (nmat == 2 || a.gemm) ? npass : 1;
  a.sh_tiles = (a0.sh_tiles + t8 * a.sh_npass - 1) / (t8 * a.sh_npass);
  a.sh_items = a.sh_tiles * ((a0.N + a.sh_chunk - 1) / a.sh_chunk);
  const long items = (long)a.sh_items + max_items;
  const int grid = items < cap ? (items > 0 ? (int)items : 1) : cap;
  a.lds_bytes = expert_lds_bytes(with_mfma, a.gemm, fmt, nmat, t8 * tr, K, max_r);
  a.max_r = max_r;
  return launch_fmt(with_mfma, fmt, nmat, tr, a, grid, s, e0, e1);
}

// The one-row down + blend where the down pass streams at most 26 MB; above
// that its time is bandwidth, which the two-kernel form streams better
// (measured on MI355X: the 25 MB BF16 Qwen3-30B-shaped row 0.8 us faster
// fused, the 28 MB MXFP4 one 1.7 us slower).  4 output columns per
// workgroup, so the h columns spread over >= 256 workgroups at h >= 1024.
bool down_blend1_plan(int fmt, int N, int h, int K, int sh_K, bool has_sh, int k, int *tr,
                      int *lds_bytes) {
  if (N != 1 || (has_sh && sh_K != K)) return false;
  const int ns = k + (has_sh ? 1 : 0);
  const double eb = fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 2 : fmt == FMT_FP8 ? 1 : 0.5;
  if ((double)ns * h * K * eb > 26.0 * (1 << 20)) return false;
  const int lb = fmt == FMT_F32 ? 4 : 2;
  const int t = 4;  // output columns per workgroup
  const long lds = (long)ns * (K * lb + 16) + (long)t * ns * 4;
  if (lds > 65536) return false;
  *tr = t;
  *lds_bytes = (int)((lds + 15) & ~15L);
  return true;
}

hipError_t launch_down_blend1(int fmt, const Down1Args &a, int lds_bytes, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1) {
  switch (fmt) {
    case FMT_F32: return launch_down_blend1_f32(a, lds_bytes, s, e0, e1);
    case FMT_BF16: return launch_down_blend1_bf16(a, lds_bytes, s, e0, e1);
    case FMT_FP8: return launch_down_blend1_fp8(a, lds_bytes, s, e0, e1);
    default: return launch_down_blend1_mxfp4(a, lds_bytes, s, e0, e1);
  }
}

// ------------------------------------------------------------------ blend

namespace {

// out[t, c] = sum_j w[t, j] * y[t k + j, c]  (slot order)  +  g_t * y_sh[t, c]
// (forward.rs: moe_weighted_sum_blend; forward_token_major.rs: the wsum/blend
// step), in fp32, then one rounding to the act dtype, or none for an fp32
// partial.  With a base (the expert-parallel combine, forward_token_major.rs:
// residual_add / moe_batched_blend after the all-reduce) the sum starts from
// base[t, c] instead of 0.  A dropped route
// (route_pos < 0) adds nothing; a zero-computation expert's slot (an id in
// [E, E + Z)) adds w * x[t, c], its input passed through.  Four columns per thread.  Every load of a
// group of 8 slots (route_pos, w and y) and of the shared expert is issued
// before the first sum, so a row costs one memory round trip per 8 slots
// rather than two per slot.
template <bool F32>
__global__ __launch_bounds__(256) void blend_kernel(BlendArgs a) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.h) return;
  const size_t r0 = (size_t)t * a.k;
  const bool sh = a.y_sh != nullptr;
  const float g = sh && a.g ? a.g[t] : 1.f;
  const f32x4 ysh = sh ? *(const f32x4 *)(a.y_sh + (size_t)t * a.h + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = a.base ? *(const f32x4 *)(a.base + (size_t)t * a.h + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  // the input row's columns, which a zero-computation expert passes through
  f32x4 xv = {0.f, 0.f, 0.f, 0.f};
  if (a.Z > 0) {
    if (a.x_f32) {
      xv = *(const f32x4 *)((const float *)a.x + (size_t)t * a.h + c);
    } else {
      const u32x2 b = *(const u32x2 *)((const uint16_t *)a.x + (size_t)t * a.h + c);
      xv = f32x4{bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y)};
    }
  }
  for (int j0 = 0; j0 < a.k; j0 += 8) {
    int p[8], e[8];
    float wj[8];
    f32x4 yv[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {  // slots past k repeat slot k-1 and are not summed
      const size_t r = r0 + min(j0 + u, a.k - 1);
      p[u] = a.route_pos[r];
      e[u] = a.Z > 0 ? a.idx[r] : -1;
      wj[u] = a.w[r];
      yv[u] = *(const f32x4 *)(a.y + r * a.h + c);
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      // a routed expert's output, or a zero expert's input row (its id past
      // the real experts: the compaction gave it no route)
      const bool on = j0 + u < a.k && p[u] >= 0;
      const bool zero = j0 + u < a.k && e[u] >= a.E && e[u] < a.E + a.Z;
      const f32x4 v = zero ? xv : yv[u];
      const f32x4 s = {fmaf(wj[u], v.x, acc.x), fmaf(wj[u], v.y, acc.y),
                       fmaf(wj[u], v.z, acc.z), fmaf(wj[u], v.w, acc.w)};
      acc = on || zero ? s : acc;
    }
  }
  if (sh) {
    acc.x = fmaf(g, ysh.x, acc.x);
    acc.y = fmaf(g, ysh.y, acc.y);
    acc.z = fmaf(g, ysh.z, acc.z);
    acc.w = fmaf(g, ysh.w, acc.w);
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

hipError_t launch_blend(bool act_f32, const BlendArgs &a, hipStream_t s, hipEvent_t e0,
                        hipEvent_t e1) {
  dim3 grid((a.h + 1023) / 1024, a.N), block(256);
  if (act_f32)
    hipExtLaunchKernelGGL(blend_kernel<true>, grid, block, 0, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL(blend_kernel<false>, grid, block, 0, s, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace moe
