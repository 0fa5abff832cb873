// Pieces shared by the bf16 tile kernels (grouped_gemm.hip: the forward's
// grouped GEMM; xgemm.hip: the backward's products with K-major operands):
// constants of the 256 x 256 x 64 tile, buffer resources, direct-to-LDS
// loads, s_waitcnt encoding, the unit plan and decoder of the device-built
// tile lists, and the bf16 / fp32 epilogue of a 128 x 128 wavefront block.
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Common pieces of the bf16 tile code.
//
// Operand pipeline.  BK = 64 (one 128-byte cache line per operand row and K
// step).  LDS stages are filled by direct-to-LDS buffer loads: each
// wavefront instruction moves 8 rows x 128 bytes straight into 1 KB of LDS,
// with no staging registers.  Rows past the segment (or past the weight
// matrix) read as zero through the buffer range check, so ragged tails need
// no clamping.
//
// LDS layout: row r of a stage occupies 128 bytes = eight 16-byte chunks;
// chunk c sits in slot c ^ g(r), g(r) = (r ^ (r >> 3)) & 7, which keeps the
// 16-byte fragment reads of 16 consecutive rows on distinct banks.
//
// Work order.  Units enumerate each list's tiles expert by expert and, inside
// one expert, N-tile by N-tile over all of its M tiles.  Each XCD (XCD =
// workgroup id % 8) takes a contiguous range of each list, so the tiles that
// share an expert's weight tile run close together on one XCD (its L2 holds
// the tile once).  When a list leaves a last, partly filled round, those last
// tiles are split along K into s parts (s = floor(grid / leftover), at least
// 4 K steps per part); the parts write fp32 partial tiles (row-major) and a
// fix-up kernel adds them in part order, so results do not depend on timing.
constexpr int kBM2 = 256, kBN2 = 256, kBK2 = 64;
constexpr int kXcds = 8;
constexpr int kStageElems = 256 * kBK2;          // one 256-row operand tile of one stage (bf16 elements)
constexpr int kMaxSplitUnits = 256;              // partial tiles the workspace holds per list
constexpr int kTileInts = 8;                     // tile entry: seg, r0, r1, first tile of seg, tiles of seg
constexpr int kBM3 = 64, kStages3 = 3;           // short-tile shape and ring depth
constexpr int kStage3Elems = (kBM3 + kBN2) * kBK2;
constexpr int kLdsElems = 2 * 2 * kStageElems > kStages3 * kStage3Elems ? 2 * 2 * kStageElems
                                                                        : kStages3 * kStage3Elems;
// voffset of a row that must read as zero in gather mode (beyond every A buffer)
constexpr int kOobOffset = 0x7fff0000;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

// 16 bytes per lane from `voff + soff` of the buffer straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// The same as a nontemporal (streaming) load: for data read once per call,
// such as the expert weights of the 64-row tiles.  Measured: decode-shape
// down projection 173 -> 145 us, up 339 -> 322 us; on the 256-row tiles,
// whose weight tiles are shared through L2, it was slower.
__device__ __forceinline__ void dma16_stream(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 2);
}

// s_waitcnt vmcnt(n), n < 64, leaving lgkmcnt / expcnt alone (gfx9 encoding: vmcnt
// bits 3:0 in bits 3:0 and bits 5:4 in bits 15:14; expcnt 6:4; lgkmcnt 11:8).
#define MOE_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
#define MOE_WAIT_VM0() __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0))

// How the units of one tile list are laid out: T tiles of KT steps; the
// first `full` tiles run whole, the remaining `rem` tiles run in s K-parts.
struct UnitPlan {
  int full, rem, s;
  __device__ __host__ int units() const { return full + rem * s; }
};

__device__ __forceinline__ UnitPlan plan_units(int T, int G, int KT) {
  UnitPlan p;
  const int rounds = T / G;
  p.rem = T - rounds * G;
  p.s = 1;
  if (p.rem > 0) {
    p.s = G / p.rem;
    if (p.s * p.rem > kMaxSplitUnits) p.s = kMaxSplitUnits / p.rem;
    if (p.s > KT / 4) p.s = KT / 4;
    if (p.s < 1) p.s = 1;
  }
  if (p.s == 1) p.rem = 0;
  p.full = T - p.rem;
  return p;
}

// One unit of work: rows [r0, r1) of segment `seg`, output columns from n0,
// K steps [kt0, kt1); slot >= 0 marks a K-part that writes partial tile `slot`.
struct Unit {
  int seg, r0, r1, n0, kt0, kt1, slot;
};

__device__ __forceinline__ Unit decode_unit(const int32_t* __restrict__ tiles, const UnitPlan& plan, int u,
                                            int n_ntiles, int KT, int cols_per_tile) {
  Unit w;
  int tile_lin;
  w.kt0 = 0;
  w.kt1 = KT;
  w.slot = -1;
  if (u < plan.full) {
    tile_lin = u;
  } else {
    const int v = u - plan.full;
    tile_lin = plan.full + v / plan.s;
    const int part = v % plan.s;
    w.kt0 = (int)((long long)KT * part / plan.s);
    w.kt1 = (int)((long long)KT * (part + 1) / plan.s);
    w.slot = v;
  }
  const int ti = tile_lin / n_ntiles;          // the expert's tiles occupy [first, first + cnt) * n_ntiles
  const int* te = tiles + 4 + kTileInts * ti;
  const int first = te[3], cnt = te[4];
  const int o = tile_lin - first * n_ntiles;
  const int j = o / cnt;
  const int i = first + o % cnt;
  const int* td = tiles + 4 + kTileInts * i;
  // readfirstlane: the tile entry is the same for every lane; saying so keeps
  // the buffer descriptors built from it in scalar registers
  w.seg = __builtin_amdgcn_readfirstlane(td[0]);
  w.r0 = __builtin_amdgcn_readfirstlane(td[1]);
  w.r1 = __builtin_amdgcn_readfirstlane(td[2]);
  w.n0 = __builtin_amdgcn_readfirstlane(j * cols_per_tile);
  w.kt0 = __builtin_amdgcn_readfirstlane(w.kt0);
  w.kt1 = __builtin_amdgcn_readfirstlane(w.kt1);
  w.slot = __builtin_amdgcn_readfirstlane(w.slot);
  return w;
}

// Gate-weighted combine in the down projection's epilogue (top-1 routing: a
// token has at most one slot, so the row holding it is the token's only
// writer).  Same arithmetic as the separate combine: Y rounded to bf16, then
// out = bf16(fma(g, Y, [residual] + [shared_y])).
struct CombineOut {
  const int32_t* perm;        // expert-order row -> slot id (= token); < 0: padding row
  const float* gates;         // [N]
  const uint16_t* residual;   // [N, Nn] or null
  const uint16_t* shared_y;   // [N, Nn] or null
  uint16_t* out;              // [N, Nn]; null: no fused combine
};

__device__ __forceinline__ void combine_store8(const CombineOut& cmb, int row, int col, int Nn, const Vec8& y) {
  const int t = cmb.perm[row];
  if (t < 0) return;
  const float g = cmb.gates[t];
  const size_t o = (size_t)t * Nn + col;
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  if (cmb.residual) {
    Vec8 r;
    r.u = *reinterpret_cast<const uint4*>(cmb.residual + o);
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = bf16_to_f32(r.e[v]);
  }
  if (cmb.shared_y) {
    Vec8 sy;
    sy.u = *reinterpret_cast<const uint4*>(cmb.shared_y + o);
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] += bf16_to_f32(sy.e[v]);
  }
  Vec8 ov;
#pragma unroll
  for (int v = 0; v < 8; ++v) ov.e[v] = f32_to_bf16(fmaf(g, bf16_to_f32(y.e[v]), acc[v]));
  *reinterpret_cast<uint4*>(cmb.out + o) = ov.u;
}

}  // namespace moe
