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

__device__ __host__ inline int swz8(int r) { return (r ^ (r >> 3)) & 7; }

// Epilogue staging layout: a wavefront's 32 x 64 fp32 block, 16 chunks of 4
// floats per row, chunk c of row r stored in slot c ^ ep_swz(r).  With rows
// of 64 floats every row starts on bank 0; the XOR spreads the accumulator
// writes (rows r and r + 4 in one instruction) and the 16-byte reads of
// every mode (4, 2 or 1 rows per 16 lanes) over all 64 banks (the up
// projection's 256-row kernel 1.4% faster at the Mixtral shape, the
// DeepSeek-V3 down projection 2.9%; identical results).
__device__ __forceinline__ int ep_swz(int r) { return (r & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 3); }
__device__ __forceinline__ int ep_at(int r, int c) { return r * 64 + (((c >> 2) ^ ep_swz(r)) << 2) + (c & 3); }

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
// s_waitcnt lgkmcnt(0): this wavefront's LDS operations complete; vmcnt and expcnt left alone.
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// How the units of one tile list are laid out: T tiles of KT steps; the
// first `full` tiles run whole, the remaining `rem` tiles run in s K-parts.
struct UnitPlan {
  int full, rem, s;
  __device__ __host__ int units() const { return full + rem * s; }
};

__device__ __host__ inline UnitPlan plan_units(int T, int G, int KT) {
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

// The units the workgroups of one XCD share: a contiguous slice of the plan's whole units and a
// contiguous slice of its K-part units (with one slice of the whole list, the parts, which come
// last, would all fall to the last XCDs, whose workgroups then run half units while the others
// run whole ones).  Workgroup q of the XCD takes every (G / 8)-th unit of the slices, q first.
struct XcdSlice {
  int f0, fc, p0, pc;
};
__device__ __host__ inline XcdSlice xcd_slice(const UnitPlan& pl, int xcd) {
  const int P = pl.rem * pl.s;
  const int fs = (pl.full + kXcds - 1) / kXcds, ps = (P + kXcds - 1) / kXcds;
  XcdSlice x;
  x.f0 = pl.full < xcd * fs ? pl.full : xcd * fs;
  x.fc = (pl.full < x.f0 + fs ? pl.full : x.f0 + fs) - x.f0;
  x.p0 = P < xcd * ps ? P : xcd * ps;
  x.pc = (P < x.p0 + ps ? P : x.p0 + ps) - x.p0;
  return x;
}
__device__ __host__ inline int xcd_unit(const UnitPlan& pl, const XcdSlice& x, int i) {
  return i < x.fc ? x.f0 + i : pl.full + x.p0 + (i - x.fc);
}

// One unit of work: rows [r0, r1) of segment `seg`, output columns from n0,
// K steps [kt0, kt1); slot >= 0 marks a K-part that writes partial tile `slot`.
// Rows [x0, x1) (x0 == x1: none) are a segment's short tail attached to a
// whole 256-row tile (tile kind 5): the unit computes them too, with the
// same weight tile.
struct Unit {
  int seg, r0, r1, n0, kt0, kt1, slot, x0, x1;
};

// Plain form of decode_unit (host-callable: the CPU tests enumerate units with it).
__device__ __host__ inline Unit decode_unit_plain(const int32_t* tiles, const UnitPlan& plan, int u, int n_ntiles,
                                                  int KT, int cols_per_tile) {
  Unit w;
  int tile_lin;
  w.kt0 = 0;
  w.kt1 = KT;
  w.slot = -1;
  w.x0 = w.x1 = 0;
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
  w.seg = td[0];
  w.r0 = td[1];
  w.r1 = td[2];
  w.n0 = j * cols_per_tile;
  return w;
}

__device__ __forceinline__ Unit decode_unit(const int32_t* __restrict__ tiles, const UnitPlan& plan, int u,
                                            int n_ntiles, int KT, int cols_per_tile) {
  Unit w = decode_unit_plain(tiles, plan, u, n_ntiles, KT, cols_per_tile);
  // readfirstlane: the tile entry is the same for every lane; saying so keeps
  // the buffer descriptors built from it in scalar registers
  w.seg = __builtin_amdgcn_readfirstlane(w.seg);
  w.r0 = __builtin_amdgcn_readfirstlane(w.r0);
  w.r1 = __builtin_amdgcn_readfirstlane(w.r1);
  w.n0 = __builtin_amdgcn_readfirstlane(w.n0);
  w.kt0 = __builtin_amdgcn_readfirstlane(w.kt0);
  w.kt1 = __builtin_amdgcn_readfirstlane(w.kt1);
  w.slot = __builtin_amdgcn_readfirstlane(w.slot);
  w.x0 = __builtin_amdgcn_readfirstlane(w.x0);
  w.x1 = __builtin_amdgcn_readfirstlane(w.x1);
  return w;
}

// fp8 64-row tile: a step loads 128 K (two 64-K halves).  A unit with an odd
// number of 64-K steps ends with a half step, whose second half lies past the
// unit's K range and, for the unit that ends at K, past the end of the row
// (the next row, or past the buffer for the last row).  The buffer range
// check covers the voffset only (the K offset travels in soffset), so those
// loads get a voffset beyond every buffer instead and read zero; the number of
// loads, which the vmcnt waits count, stays the same.
//   A (bf16 rows, one load per half hf): the half step's hf = 1 loads.
//   B (fp8 rows, 16-byte chunk `chunk` of the 128-byte step): chunks 4..7.
__device__ __host__ inline int fp8_a_voff(int voff, int hf, bool half) { return (half && hf) ? kOobOffset : voff; }
__device__ __host__ inline int fp8_b_voff(int voff, int chunk, bool half) {
  return (half && chunk >= 4) ? kOobOffset : voff;
}

// ---------------------------------------------------------------------------
// Per-segment tile table of the forward grouped GEMM.  Segment e (rows
// [off[e], off[e+1])) is cut into 256-row tiles (kind 0: floor(rows / 256),
// plus one more when at least kBigTailMin rows remain; kind 1: none; kind 2:
// as kind 0, but a segment of at least 256 rows puts its whole tail in one
// more 256-row tile; kinds 3, 4: kind 0 or 2 by choose_tail_kind) and
// 64-row tiles for the rest; pb / ps are the exclusive prefix counts of the two
// kinds over the segments.  Every workgroup builds the table in LDS from the
// offsets (E <= 256, one wavefront) and decodes its units from it, so no
// separate launch has to write a tile list first.  Unit order as for the tile
// lists: segment by segment, column tile by column tile over the segment's
// row tiles.
constexpr int kBigTailMin = 128;

struct SegTable {
  int off[kMaxExperts + 1];
  int pb[kMaxExperts + 1];
  int ps[kMaxExperts + 1];
  int kind;   // the tile kind the table was built for (kinds 3 and 4 resolved)
};

// Kind 5: kind 0, except that a segment of at least 256 rows whose tail is
// shorter than kBigTailMin attaches up to 32 tail rows to each of its whole
// 256-row tiles (attach_rows of them in all, 32 to each of the first tiles);
// only the rest of the tail goes to 64-row tiles.
constexpr int kAttachRows = 32;
// The forward 256-row kernel's stage: A rows 0..255 of the tile and 256..287 for attached rows, then the
// 256 B rows; its K-part partial tiles have kBM2P rows (the attached ones at 256..287).
constexpr int kARows = 256 + kAttachRows;
constexpr int kStageA = kARows * 64;
constexpr int kStage2 = (kARows + 256) * 64;
constexpr int kBM2P = kARows;
__device__ __host__ inline int attach_rows(int rows) {
  const int nb = rows / 256, rest = rows - 256 * nb;
  return rest < kBigTailMin ? (rest < kAttachRows * nb ? rest : kAttachRows * nb) : 0;
}
constexpr int kSegTableElems = (int)((sizeof(SegTable) + 15) / 16) * 8;   // in 16-bit LDS elements
// The forward 256-row kernel's LDS: two operand stages, the tile table, then a tail that stages
// the attached rows' outputs (32 rows x (256 + 8) bf16, or 4 x 1024 fp32).
constexpr int kTailOff = ((2 * kStage2 + kSegTableElems + 127) / 128) * 128;
constexpr int kTailElems = 32 * (256 + 8);
static_assert(kTailOff + kTailElems <= 80 * 1024, "the 256-row kernel's LDS fits 160 KB");

__device__ __host__ inline void seg_tiles(int rows, int kind, int& nb, int& ns) {
  nb = kind == 1 ? 0 : rows / 256;
  int rest = rows - nb * 256;
  if (((kind == 0 || kind == 5) && rest >= kBigTailMin) ||
      (kind == 2 && rest > 0 && (nb > 0 || rest >= kBigTailMin))) {
    nb += 1;
    rest = 0;
  }
  if (kind == 5) rest -= attach_rows(rows);
  ns = rest > 0 ? (rest + 63) / 64 : 0;
}

// Kinds 3 (up projection) and 4 (down projection) choose between kind 0 and
// kind 2 from the segment sizes, the same way in every workgroup.  Kind 2
// moves the short tails of long segments from the 64-row kernel, which
// streams the expert's weights again for them, into 256-row units that find
// those weights in L2, at the price of more 256-row units, all of which a
// workgroup runs in turn.  Taken when that adds no round of 256-row units
// (ceil(T2 / G) = ceil(T0 / G)), or, for a down projection, when the 256-row
// units already take 8 or more rounds.  (Measured: DeepSeek-V3 down projection
// 2.76 -> 2.68 ms, the Switch shape's up and down 3% faster each; Mixtral's
// down projection 0.89 -> 1.21 ms and the DeepSeek-V3 and Mixtral up
// projections 2-3% slower with kind 2, and the rule keeps kind 0 for them.)
__device__ __host__ inline int choose_tail_kind(long long t0, long long t2, int G, bool down) {
  const long long r0 = (t0 + G - 1) / G, r2 = (t2 + G - 1) / G;
  return (r2 == r0 || (down && t0 >= 8LL * G)) ? 2 : 0;
}

// Called by every thread of the workgroup; wavefront 0 fills the table (lane l
// takes segments 4l .. 4l + 3), then a barrier.  n_ntiles and G (the grid)
// serve kinds 3 and 4 only; with `attach`, kind 0 (given or chosen) becomes 5.
__device__ __forceinline__ void build_seg_table(SegTable& t, const int32_t* __restrict__ offsets, int n_seg,
                                                int dense_rows, int kind, int n_ntiles = 0, int G = 1,
                                                bool attach = false) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int o[4], rows[4], nb[4], ns[4], sb = 0, ss = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      int lo = 0, hi = 0;
      if (e < n_seg) {
        lo = offsets ? offsets[e] : 0;
        hi = offsets ? offsets[e + 1] : dense_rows;
      }
      o[i] = lo;
      rows[i] = hi - lo;
    }
    if (kind >= 3) {
      int c0 = 0, c2 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int b0, b2, s_;
        seg_tiles(rows[i], 0, b0, s_);
        seg_tiles(rows[i], 2, b2, s_);
        c0 += b0;
        c2 += b2;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        c0 += __shfl_xor(c0, d);
        c2 += __shfl_xor(c2, d);
      }
      kind = choose_tail_kind((long long)c0 * n_ntiles, (long long)c2 * n_ntiles, G, kind == 4);
    }
    if (attach && kind == 0) kind = 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      seg_tiles(rows[i], kind, nb[i], ns[i]);
      if (4 * lane + i >= n_seg) nb[i] = ns[i] = 0;
      sb += nb[i];
      ss += ns[i];
    }
    int ib = sb, is = ss;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int vb = __shfl_up(ib, d), vs = __shfl_up(is, d);
      if (lane >= d) { ib += vb; is += vs; }
    }
    int eb = ib - sb, es = is - ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < n_seg) {
        t.off[e] = o[i];
        t.pb[e] = eb;
        t.ps[e] = es;
      }
      eb += nb[i];
      es += ns[i];
    }
    if (lane == 63) {
      t.off[n_seg] = n_seg > 0 ? (offsets ? offsets[n_seg] : dense_rows) : 0;
      t.pb[n_seg] = ib;
      t.ps[n_seg] = is;
      t.kind = kind;
    }
  }
  __syncthreads();
}

// Unit u of the 256-row (big) or 64-row list: the segment is the last one whose
// prefix count is at most the unit's tile index (binary search).
__device__ __host__ inline Unit decode_unit_seg(const SegTable& t, int n_seg, bool big, const UnitPlan& plan, int u,
                                                int n_ntiles, int KT, int cols_per_tile) {
  Unit w;
  int tile_lin;
  w.kt0 = 0;
  w.kt1 = KT;
  w.slot = -1;
  w.x0 = w.x1 = 0;
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
  const int* pre = big ? t.pb : t.ps;
  const int ti = tile_lin / n_ntiles;
  int lo = 0, hi = n_seg - 1;           // largest e with pre[e] <= ti
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= ti) lo = mid; else hi = mid - 1;
  }
  const int seg = lo, first = pre[seg], cnt = pre[seg + 1] - first;
  const int o = tile_lin - first * n_ntiles;
  const int j = o / cnt;
  // kind 5: the M tiles of column tile j are rotated by j + j cnt / 32, so that
  // the tiles carrying attached rows (the first ones) are spread over the
  // workgroups: those of an XCD take every 32nd unit of its span, which with
  // cnt dividing 32 is the same M position at every column tile, and the
  // j cnt / 32 term moves that position by one from one of them to the next
  const int m = t.kind == 5 ? (o % cnt + j + j * cnt / 32) % cnt : o % cnt;
  const int seg_lo = t.off[seg], seg_hi = t.off[seg + 1];
  w.seg = seg;
  const int xa = t.kind == 5 ? attach_rows(seg_hi - seg_lo) : 0;
  if (big) {
    w.r0 = seg_lo + m * 256;
    w.r1 = seg_hi < w.r0 + 256 ? seg_hi : w.r0 + 256;
    if (m * kAttachRows < xa) {
      const int nbig = t.pb[seg + 1] - t.pb[seg];
      w.x0 = seg_lo + nbig * 256 + m * kAttachRows;
      w.x1 = w.x0 + (xa - m * kAttachRows < kAttachRows ? xa - m * kAttachRows : kAttachRows);
    }
  } else {
    const int nbig = t.pb[seg + 1] - t.pb[seg];
    const int split = seg_hi < seg_lo + nbig * 256 + xa ? seg_hi : seg_lo + nbig * 256 + xa;
    w.r0 = split + m * 64;
    w.r1 = seg_hi < w.r0 + 64 ? seg_hi : w.r0 + 64;
  }
  w.n0 = j * cols_per_tile;
  return w;
}

__device__ __forceinline__ Unit decode_unit_lds(const SegTable& t, int n_seg, bool big, const UnitPlan& plan, int u,
                                                int n_ntiles, int KT, int cols_per_tile) {
  Unit w = decode_unit_seg(t, n_seg, big, plan, u, n_ntiles, KT, cols_per_tile);
  w.seg = __builtin_amdgcn_readfirstlane(w.seg);
  w.r0 = __builtin_amdgcn_readfirstlane(w.r0);
  w.r1 = __builtin_amdgcn_readfirstlane(w.r1);
  w.n0 = __builtin_amdgcn_readfirstlane(w.n0);
  w.kt0 = __builtin_amdgcn_readfirstlane(w.kt0);
  w.kt1 = __builtin_amdgcn_readfirstlane(w.kt1);
  w.slot = __builtin_amdgcn_readfirstlane(w.slot);
  w.x0 = __builtin_amdgcn_readfirstlane(w.x0);
  w.x1 = __builtin_amdgcn_readfirstlane(w.x1);
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
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = fmaf(g, bf16_to_f32(y.e[v]), acc[v]);
  *reinterpret_cast<uint4*>(cmb.out + o) = pack_bf16x8(acc);
}

}  // namespace moe
