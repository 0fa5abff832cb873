// Grouped expert GEMM over ragged per-expert row segments.
//
// [L] "Concept / FFN swap": every expert is an independent feed-forward
// network, usually SwiGLU; [G] "How an MoE layer works": experts share one
// architecture; [X] "Future of expert parallelism": grouped GEMMs that batch
// many experts in one launch.  Rows [offsets[e], offsets[e+1]) of the
// expert-sorted activations go through expert e.
//
// Work decomposition.  A one-workgroup kernel turns `offsets` into a list of
// (expert, row_begin, row_end) tiles of at most BM rows on the device, so the
// host never waits for the routing result.  The GEMM grid is sized for the
// worst case (ceil(rows / BM) + E tiles); workgroups past the real tile count
// exit at once.
//
// Tile kernel (bf16 in, fp32 accumulate): 256 threads = 4 wavefronts in a 2x2
// layout over a BM x BN = 128 x 128 output tile, BK = 64, operands staged
// through double-buffered LDS with rows padded by 16 bytes, fragments fed to
// v_mfma_f32_32x32x16_bf16 (each wavefront: 2x2 MFMA blocks of 32x32).
//   SwiGLU up : the B tile holds 64 rows of W1 and the same 64 rows of W3, and
//               each wavefront owns matching W1/W3 column blocks, so the
//               epilogue forms SiLU(a1) * a3 in registers and writes bf16 H.
//   GELU up   : GELU(acc + b1) -> bf16 H.
//   down      : acc (+ b2) -> bf16 Y.
//
// MFMA 32x32x16 layout (lane l): A row l%32, k = 8*(l/32)..+7; B column l%32,
// same k; D column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#include "moe_internal.h"

namespace moe {


// Splits every segment into 256-row tiles and 64-row tiles: floor(rows / 256)
// full tiles, one more 256-row tile when at least kBigTailMin rows remain,
// otherwise ceil(rest / 64) 64-row tiles.  Each list: [0] = tile count; tile i
// at [4 + 8 i] = (segment, row_begin, row_end, first tile of the segment in
// this list, tiles of the segment in this list, 0, 0, 0).
constexpr int kBigTailMin = 128;

__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets, int n_seg,
                                                          int dense_rows, int32_t* __restrict__ big,
                                                          int max_big, int32_t* __restrict__ small,
                                                          int max_small) {
  __shared__ int tot_b[4], tot_s[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int lo = 0, hi = 0, nb = 0, ns = 0, split = 0;
  if (tid < n_seg) {
    lo = offsets ? offsets[tid] : 0;
    hi = offsets ? offsets[tid + 1] : dense_rows;
    const int rows = hi - lo;
    nb = rows / 256;
    const int rest = rows - nb * 256;
    if (rest >= kBigTailMin) { nb += 1; }
    else { ns = (rest + 63) / 64; }
    split = min(hi, lo + nb * 256);
  }
  int ib = nb, is = ns;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int vb = __shfl_up(ib, off), vs = __shfl_up(is, off);
    if (lane >= off) { ib += vb; is += vs; }
  }
  if (lane == 63) { tot_b[wave] = ib; tot_s[wave] = is; }
  __syncthreads();
  int base_b = ib - nb, base_s = is - ns;
  for (int w = 0; w < wave; ++w) { base_b += tot_b[w]; base_s += tot_s[w]; }
  for (int i = 0; i < nb; ++i) {
    const int id = base_b + i;
    if (id >= max_big) break;
    int4* e = reinterpret_cast<int4*>(big + 4 + 8 * id);
    e[0] = int4{tid, lo + i * 256, min(hi, lo + (i + 1) * 256), base_b};
    e[1] = int4{nb, 0, 0, 0};
  }
  for (int i = 0; i < ns; ++i) {
    const int id = base_s + i;
    if (id >= max_small) break;
    int4* e = reinterpret_cast<int4*>(small + 4 + 8 * id);
    e[0] = int4{tid, split + i * 64, min(hi, split + (i + 1) * 64), base_s};
    e[1] = int4{ns, 0, 0, 0};
  }
  if (tid == 0) {
    big[0] = min(tot_b[0] + tot_b[1] + tot_b[2] + tot_b[3], max_big);
    small[0] = min(tot_s[0] + tot_s[1] + tot_s[2] + tot_s[3], max_small);
  }
}

// ---------------------------------------------------------------------------
// 256 x 256 tile, persistent, XCD-aware (the routed-expert and shared-expert
// GEMMs of prefill-sized batches).
//
// 256 threads = 4 wavefronts in a 2x2 layout; each wavefront owns a 128 x 128
// block = 4 x 4 MFMA 32x32x16 blocks whose 256 fp32 accumulators per lane
// live in AGPRs (one workgroup per CU).
//
// Operand pipeline.  BK = 64 (one 128-byte cache line per operand row and K
// step); two 64 KB LDS stages are filled by direct-to-LDS buffer loads (each
// wavefront instruction moves 8 rows x 128 bytes straight into 1 KB of LDS,
// no staging registers).  The loads for step k+1 are issued in slices
// between the MFMAs of the first three sub-steps of step k, and the fragments of each 16-wide sub-step
// are read from LDS while the previous sub-step's 16 MFMAs issue.  One
// fence-free barrier per step.  Rows past the segment (or past the weight
// matrix) read as zero, so ragged tails need no clamping.
//
// LDS layout: row r of a stage occupies 128 bytes = eight 16-byte chunks;
// chunk c sits in slot c ^ g(r), g(r) = (r ^ (r >> 3)) & 7, which keeps the
// 16-byte fragment reads of 16 consecutive rows on distinct banks.
//
// Work order.  Units enumerate the tiles expert by expert and, inside one
// expert, N-tile by N-tile over all of its M tiles, so the workgroups running
// together on one XCD (XCD = workgroup id % 8; each XCD walks a contiguous
// range of units) share that expert's weight tile and A rows in their L2.
// When the tile count leaves a last, partly filled round, those last tiles
// are split along K into s parts (s = floor(grid / leftover)); the parts
// write fp32 partial tiles and a fix-up kernel adds them in part order, so
// results do not depend on timing.
constexpr int kBM2 = 256, kBN2 = 256, kBK2 = 64;
constexpr int kXcds = 8;
constexpr int kStageElems = 256 * kBK2;          // one operand tile of one stage (bf16 elements)
constexpr int kMaxSplitUnits = 256;              // partial tiles the workspace holds
constexpr int kTileInts = 8;                     // tile entry: seg, r0, r1, first tile of seg, tiles of seg

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

union Vec8 {
  uint4 u;
  uint16_t e[8];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

// 16 bytes per lane from `voff + soff` of the buffer straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(0) leaving lgkmcnt / expcnt alone (gfx9 encoding).
#define MOE_WAIT_VM0() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))

// How the units of a grouped GEMM are laid out: T tiles of KT steps; the
// first `full` tiles run whole, the remaining `rem` tiles run in s K-parts.
struct UnitPlan {
  int full, rem, s;
  __device__ __host__ int units() const { return full + rem * s; }
};

__device__ __forceinline__ UnitPlan plan_units(int T, int G) {
  UnitPlan p;
  const int rounds = T / G;
  p.rem = T - rounds * G;
  p.s = 1;
  if (p.rem > 0) {
    p.s = G / p.rem;
    if (p.s * p.rem > kMaxSplitUnits) p.s = kMaxSplitUnits / p.rem;
    if (p.s < 1) p.s = 1;
  }
  if (p.s == 1) p.rem = 0;
  p.full = T - p.rem;
  return p;
}

// Epilogue of one 128 x 128 wavefront block (rows r0 + wm*128 .., columns of
// the output n0 ..): activation, bias, bf16 rounding, 16-byte stores.
// `ep` is this wavefront's 16 KB of LDS; `src_acc` the accumulators.
template <int MODE, bool HAS_BIAS>
__device__ __forceinline__ void store_block(f32x16 (&acc)[4][4], float* ep, int lane, int kh, int l32, int wm,
                                            int wn, int r0, int r1, int n0, int Nn, int seg,
                                            const uint16_t* __restrict__ bias, uint16_t* __restrict__ out) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[((r >> 2) * 8 + kh * 4 + (r & 3)) * 128 + ni * 32 + l32] = acc[mi][ni][r];
    __builtin_amdgcn_wave_barrier();
    const int rbase = r0 + wm * 128 + mi * 32;
    if (MODE == MODE_SWIGLU_UP) {
      // cols 0..63 hold x W1^T, cols 64..127 the matching x W3^T
#pragma unroll 1
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const int row = rbase + rr, col = n0 + wn * 64 + c8;
        if (row < r1 && col < Nn) {
          const float* src = ep + rr * 128 + c8;
          Vec8 o;
#pragma unroll
          for (int v = 0; v < 8; ++v) o.e[v] = f32_to_bf16(silu_f(src[v]) * src[64 + v]);
          *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = o.u;
        }
      }
    } else {
#pragma unroll 1
      for (int pass = 0; pass < 8; ++pass) {
        const int rr = pass * 4 + (lane >> 4), c8 = (lane & 15) * 8;
        const int row = rbase + rr, col = n0 + wn * 128 + c8;
        if (row < r1 && col < Nn) {
          const float* src = ep + rr * 128 + c8;
          Vec8 b;
          if (HAS_BIAS) b.u = *reinterpret_cast<const uint4*>(bias + (size_t)seg * Nn + col);
          Vec8 o;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            float x = src[v];
            if (HAS_BIAS) x += bf16_to_f32(b.e[v]);
            if (MODE == MODE_GELU_UP) x = gelu_f(x);
            o.e[v] = f32_to_bf16(x);
          }
          *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = o.u;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256, 1) void grouped_gemm_256_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ tiles, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    float* __restrict__ partials, int K, int Nn, int n_ntiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * kStageElems];

  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int T_m = tiles[0];
  const int G = gridDim.x;
  const UnitPlan plan = plan_units(T_m * n_ntiles, G);
  const int U = plan.units();
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  const int span = (U + kXcds - 1) / kXcds;
  const int u_end = min(U, (xcd + 1) * span);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps buffer descriptors scalar
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const size_t wstride = (size_t)Nn * K;
  const int rowbytes = K * 2;
  const int KT = K / kBK2;

  // DMA: wavefront w fills rows 64w..64w+63 of both operands, 8 rows per
  // instruction; lane -> row (lane >> 3), slot lane & 7 holding chunk slot ^ g(row).
  int voff[8], voffb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 64 * wave + 8 * u + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);
    voff[u] = row * rowbytes + chunk * 16;
    // SwiGLU: wavefronts 2 and 3 fill B rows 128..255 from W3, whose rows restart at 0
    voffb[u] = (MODE == MODE_SWIGLU_UP ? (row & 127) : row) * rowbytes + chunk * 16;
  }
  // Fragment reads: row r = base + 32 x + l32 (base a multiple of 128), chunk
  // c = 2 kk + kh; g(r) = g(l32) ^ 4 (x & 1), so slot = (2 kk) ^ h ^ 4 (x & 1).
  const int h = kh ^ swz8(l32);
  const int abase = (wm * 128 + l32) * kBK2;
  const int bbase = kStageElems + (MODE == MODE_SWIGLU_UP ? (wn * 64 + l32) : (wn * 128 + l32)) * kBK2;

  for (int u = xcd * span + q; u < u_end; u += per_xcd) {
    // unit -> (M tile i, N tile j, K range)
    int tile_lin, kt0 = 0, kt1 = KT, part = -1;
    if (u < plan.full) {
      tile_lin = u;
    } else {
      const int v = u - plan.full;
      tile_lin = plan.full + v / plan.s;
      part = v % plan.s;
      kt0 = (int)((long long)KT * part / plan.s);
      kt1 = (int)((long long)KT * (part + 1) / plan.s);
    }
    const int ti = tile_lin / n_ntiles;          // the expert's tiles occupy [first, first + cnt) * n_ntiles
    const int* te = tiles + 4 + kTileInts * ti;
    const int first = te[3], cnt = te[4];
    const int o = tile_lin - first * n_ntiles;
    const int j = o / cnt;
    const int i = first + o % cnt;
    const int* td = tiles + 4 + kTileInts * i;
    const int seg = td[0], r0 = td[1], r1 = td[2];
    const int n0 = j * cols_per_tile;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)r0 * K, (uint32_t)(r1 - r0) * rowbytes);
    const int nb_rows = min(cols_per_tile, Nn - n0);
    const uint16_t* wsrc = (MODE == MODE_SWIGLU_UP && wave >= 2) ? W3 : W;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(wsrc + (size_t)seg * wstride + (size_t)n0 * K, (uint32_t)nb_rows * rowbytes);

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    if (kt0 < kt1) {  // prologue: step kt0 into stage kt0 & 1 (a K-part can be empty)
      uint16_t* st = lds + (kt0 & 1) * (2 * kStageElems);
      const int so = kt0 * kBK2 * 2;
#pragma unroll
      for (int uu = 0; uu < 8; ++uu) {
        dma16(ra, st + (64 * wave + 8 * uu) * kBK2, voff[uu], so);
        dma16(rb, st + kStageElems + (64 * wave + 8 * uu) * kBK2, voffb[uu], so);
      }
    }
    for (int kt = kt0; kt < kt1; ++kt) {
      MOE_WAIT_VM0();                      // this wavefront's loads of step kt have landed
      __builtin_amdgcn_s_barrier();        // ... and everyone's; stage kt+1 is free again
      const uint16_t* st = lds + (kt & 1) * (2 * kStageElems);
      uint16_t* nx = lds + ((kt + 1) & 1) * (2 * kStageElems);
      const bool more = kt + 1 < kt1;
      const int so = (kt + 1) * kBK2 * 2;
      bf16x8 fa[2][4], fb[2][4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int sw = (h ^ (4 * (x & 1))) << 3;
        fa[0][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + sw);
        fb[0][x] = *reinterpret_cast<const bf16x8*>(
            st + bbase + (MODE == MODE_SWIGLU_UP ? (x >> 1) * 8192 + (x & 1) * 2048 : 2048 * x) + sw);
      }
#pragma unroll
      for (int kk = 0; kk < kBK2 / 16; ++kk) {
        const int c = kk & 1;
        if (more && kk < 3) {
          // slices 3 / 3 / 2 over the first three sub-steps: the last slice still has a
          // quarter step of MFMAs to land before the wait at the top of the next step
#pragma unroll
          for (int uu = 3 * kk; uu < 3 * kk + 3; ++uu) {
            if (uu < 8) {
              dma16(ra, nx + (64 * wave + 8 * uu) * kBK2, voff[uu], so);
              dma16(rb, nx + kStageElems + (64 * wave + 8 * uu) * kBK2, voffb[uu], so);
            }
          }
        }
        if (kk + 1 < kBK2 / 16) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int sw = (h ^ (4 * (x & 1)) ^ (2 * (kk + 1))) << 3;
            fa[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + sw);
            fb[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(
                st + bbase + (MODE == MODE_SWIGLU_UP ? (x >> 1) * 8192 + (x & 1) * 2048 : 2048 * x) + sw);
          }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // 4 MFMA
        }
      }
    }
    __syncthreads();   // every wavefront is done with the stages before the epilogue reuses them

    if (part < 0) {
      float* ep = reinterpret_cast<float*>(lds) + wave * (32 * 128);
      store_block<MODE, HAS_BIAS>(acc, ep, lane, kh, l32, wm, wn, r0, r1, n0, Nn, seg, bias, out);
    } else {
      // fp32 partial tile, layout [part unit][256 rows][256 accumulator columns] in MFMA order
      float* dst = partials + (size_t)(u - plan.full) * (kBM2 * kBN2) + (size_t)wave * (128 * 128 * 4 / 4);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          *reinterpret_cast<f32x16*>(dst + ((mi * 4 + ni) * 64 + lane) * 16) = acc[mi][ni];
    }
    __syncthreads();   // the next unit's first loads must not overtake this epilogue
  }
}

// Adds the K-parts of each split tile in part order and runs the epilogue.
// One workgroup per split tile (grid = kMaxSplitUnits; extra workgroups exit).
template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256, 1) void split_fixup_kernel(const int32_t* __restrict__ tiles,
                                                             const float* __restrict__ partials,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ out, int Nn, int n_ntiles,
                                                             int G) {
  __shared__ __attribute__((aligned(1024))) float lds[4 * 32 * 128];
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int T_m = tiles[0];
  const UnitPlan plan = plan_units(T_m * n_ntiles, G);
  const int t = blockIdx.x;
  if (t >= plan.rem) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, kh = lane >> 5;
  const int tile_lin = plan.full + t;
  const int ti = tile_lin / n_ntiles;
  const int* te = tiles + 4 + kTileInts * ti;
  const int first = te[3], cnt = te[4];
  const int o = tile_lin - first * n_ntiles;
  const int j = o / cnt;
  const int i = first + o % cnt;
  const int* td = tiles + 4 + kTileInts * i;
  const int seg = td[0], r0 = td[1], r1 = td[2];
  const int n0 = j * cols_per_tile;
  f32x16 acc[4][4];
  for (int p = 0; p < plan.s; ++p) {
    const float* src = partials + (size_t)(t * plan.s + p) * (kBM2 * kBN2) + (size_t)wave * (128 * 128);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const f32x16 v = *reinterpret_cast<const f32x16*>(src + ((mi * 4 + ni) * 64 + lane) * 16);
        acc[mi][ni] = p == 0 ? v : acc[mi][ni] + v;
      }
  }
  store_block<MODE, HAS_BIAS>(acc, lds + wave * (32 * 128), lane, kh, l32, wm, wn, r0, r1, n0, Nn, seg, bias, out);
}

// ---------------------------------------------------------------------------
// 64 x 256 tile for short segments (decode batches, experts with few routed
// rows, the tails of long segments): there the GEMM streams the expert's
// weights for a handful of rows, so the design goal is many bytes in flight
// per CU rather than MFMA reuse.  4 wavefronts in a 1 x 4 layout, each 64 x 64
// (2 x 2 MFMA 32x32x16 blocks); a 3-stage LDS ring of 40 KB stages (A: 64 rows,
// B: 256 rows, 128 bytes each) keeps two K steps of loads in flight.  Same
// direct-to-LDS loads, swizzle, work order and K-split tail as the 256-row
// kernel.
constexpr int kBM3 = 64, kStages3 = 3;
constexpr int kStage3Elems = (kBM3 + kBN2) * kBK2;

template <int MODE, bool HAS_BIAS>
__device__ __forceinline__ void store_block64(f32x16 (&acc)[2][2], float* ep, int lane, int kh, int l32, int wn,
                                              int r0, int r1, int n0, int Nn, int seg,
                                              const uint16_t* __restrict__ bias, uint16_t* __restrict__ out) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[((r >> 2) * 8 + kh * 4 + (r & 3)) * 64 + ni * 32 + l32] = acc[mi][ni][r];
    __builtin_amdgcn_wave_barrier();
    const int rbase = r0 + mi * 32;
    if (MODE == MODE_SWIGLU_UP) {
      // cols 0..31 hold x W1^T, cols 32..63 the matching x W3^T
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) {
        const int rr = pass * 16 + (lane >> 2), c8 = (lane & 3) * 8;
        const int row = rbase + rr, col = n0 + wn * 32 + c8;
        if (row < r1 && col < Nn) {
          const float* src = ep + rr * 64 + c8;
          Vec8 o;
#pragma unroll
          for (int v = 0; v < 8; ++v) o.e[v] = f32_to_bf16(silu_f(src[v]) * src[32 + v]);
          *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = o.u;
        }
      }
    } else {
#pragma unroll 1
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const int row = rbase + rr, col = n0 + wn * 64 + c8;
        if (row < r1 && col < Nn) {
          const float* src = ep + rr * 64 + c8;
          Vec8 b;
          if (HAS_BIAS) b.u = *reinterpret_cast<const uint4*>(bias + (size_t)seg * Nn + col);
          Vec8 o;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            float x = src[v];
            if (HAS_BIAS) x += bf16_to_f32(b.e[v]);
            if (MODE == MODE_GELU_UP) x = gelu_f(x);
            o.e[v] = f32_to_bf16(x);
          }
          *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = o.u;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256, 1) void grouped_gemm_64_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ tiles, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    float* __restrict__ partials, int K, int Nn, int n_ntiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages3 * kStage3Elems];

  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int T_m = tiles[0];
  const int G = gridDim.x;
  const UnitPlan plan = plan_units(T_m * n_ntiles, G);
  const int U = plan.units();
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  const int span = (U + kXcds - 1) / kXcds;
  const int u_end = min(U, (xcd + 1) * span);

  const int tid = threadIdx.x;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);     // wavefront = column block
  const int lane = tid & 63;
  const int l32 = lane & 31, kh = lane >> 5;
  const size_t wstride = (size_t)Nn * K;
  const int rowbytes = K * 2;
  const int KT = K / kBK2;

  // DMA: wavefront w fills A rows 16w..16w+15 (2 instructions) and B rows 64w..64w+63 (8).
  int voffa[2], voffb[8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * wn + 8 * u + (lane >> 3);
    voffa[u] = row * rowbytes + (((lane & 7) ^ swz8(row)) * 16);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 64 * wn + 8 * u + (lane >> 3);
    voffb[u] = (MODE == MODE_SWIGLU_UP ? (row & 127) : row) * rowbytes + (((lane & 7) ^ swz8(row)) * 16);
  }
  // Fragment reads: A row 32 mi + l32 -> g = swz8(l32) ^ 4 mi; B rows: SwiGLU W1 / W3 rows
  // (128 ni) + 32 wn + l32 -> g = swz8(l32) ^ 4 (wn & 1); otherwise 64 wn + 32 ni + l32 -> ^ 4 ni.
  const int h = kh ^ swz8(l32);
  const int brow0 = MODE == MODE_SWIGLU_UP ? (32 * wn + l32) : (64 * wn + l32);
  const int bstep = MODE == MODE_SWIGLU_UP ? 128 : 32;
  const int hb0 = MODE == MODE_SWIGLU_UP ? (h ^ (4 * (wn & 1))) : h;
  const int hb1 = MODE == MODE_SWIGLU_UP ? hb0 : (h ^ 4);

  for (int u = xcd * span + q; u < u_end; u += per_xcd) {
    int tile_lin, kt0 = 0, kt1 = KT, part = -1;
    if (u < plan.full) {
      tile_lin = u;
    } else {
      const int v = u - plan.full;
      tile_lin = plan.full + v / plan.s;
      part = v % plan.s;
      kt0 = (int)((long long)KT * part / plan.s);
      kt1 = (int)((long long)KT * (part + 1) / plan.s);
    }
    const int ti = tile_lin / n_ntiles;
    const int* te = tiles + 4 + kTileInts * ti;
    const int first = te[3], cnt = te[4];
    const int o = tile_lin - first * n_ntiles;
    const int j = o / cnt;
    const int i = first + o % cnt;
    const int* td = tiles + 4 + kTileInts * i;
    const int seg = td[0], r0 = td[1], r1 = td[2];
    const int n0 = j * cols_per_tile;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)r0 * K, (uint32_t)(r1 - r0) * rowbytes);
    const int nb_rows = min(cols_per_tile, Nn - n0);
    const uint16_t* wsrc = (MODE == MODE_SWIGLU_UP && wn >= 2) ? W3 : W;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(wsrc + (size_t)seg * wstride + (size_t)n0 * K, (uint32_t)nb_rows * rowbytes);

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    // prologue: steps kt0 and kt0 + 1
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kt = kt0 + p;
      if (kt < kt1) {
        uint16_t* st = lds + (kt % kStages3) * kStage3Elems;
        const int so = kt * kBK2 * 2;
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) dma16(ra, st + (16 * wn + 8 * uu) * kBK2, voffa[uu], so);
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) dma16(rb, st + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
      }
    }
    for (int kt = kt0; kt < kt1; ++kt) {
      // outstanding in issue order: step kt, then step kt + 1 (10 loads) if it exists
      if (kt + 1 < kt1) __builtin_amdgcn_s_waitcnt(10 | (7 << 4) | (15 << 8));
      else MOE_WAIT_VM0();
      __builtin_amdgcn_s_barrier();          // step kt landed everywhere; the slot of kt - 1 is free
      const uint16_t* st = lds + (kt % kStages3) * kStage3Elems;
      uint16_t* nx = lds + ((kt + 2) % kStages3) * kStage3Elems;
      const bool more = kt + 2 < kt1;
      const int so = (kt + 2) * kBK2 * 2;
      bf16x8 fa[2][2], fb[2][2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        fa[0][x] = *reinterpret_cast<const bf16x8*>(st + (32 * x + l32) * kBK2 + ((h ^ (4 * x)) << 3));
        fb[0][x] = *reinterpret_cast<const bf16x8*>(st + (kBM3 + brow0 + bstep * x) * kBK2 + ((x ? hb1 : hb0) << 3));
      }
#pragma unroll
      for (int kk = 0; kk < kBK2 / 16; ++kk) {
        const int c = kk & 1;
        if (more && kk < 3) {
          // 10 loads over the first three sub-steps: 4 / 3 / 3
          if (kk == 0) {
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) dma16(ra, nx + (16 * wn + 8 * uu) * kBK2, voffa[uu], so);
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) dma16(rb, nx + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
          } else {
#pragma unroll
            for (int uu = 3 * kk - 1; uu < 3 * kk + 2; ++uu)
              dma16(rb, nx + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
          }
        }
        if (kk + 1 < kBK2 / 16) {
          const int k2 = 2 * (kk + 1);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            fa[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(st + (32 * x + l32) * kBK2 + ((h ^ (4 * x) ^ k2) << 3));
            fb[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(
                st + (kBM3 + brow0 + bstep * x) * kBK2 + (((x ? hb1 : hb0) ^ k2) << 3));
          }
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
      }
    }
    __syncthreads();   // every wavefront is done with the ring before the epilogue reuses it

    if (part < 0) {
      float* ep = reinterpret_cast<float*>(lds) + wn * (32 * 64);
      store_block64<MODE, HAS_BIAS>(acc, ep, lane, kh, l32, wn, r0, r1, n0, Nn, seg, bias, out);
    } else {
      float* dst = partials + (size_t)(u - plan.full) * (kBM3 * kBN2) + (size_t)wn * (64 * 64);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          *reinterpret_cast<f32x16*>(dst + ((mi * 2 + ni) * 64 + lane) * 16) = acc[mi][ni];
    }
    __syncthreads();   // the next unit's first loads must not overtake this epilogue
  }
}

template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256, 1) void split_fixup64_kernel(const int32_t* __restrict__ tiles,
                                                               const float* __restrict__ partials,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ out, int Nn, int n_ntiles,
                                                               int G) {
  __shared__ __attribute__((aligned(1024))) float lds[4 * 32 * 64];
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int T_m = tiles[0];
  const UnitPlan plan = plan_units(T_m * n_ntiles, G);
  const int t = blockIdx.x;
  if (t >= plan.rem) return;
  const int tid = threadIdx.x;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, kh = lane >> 5;
  const int tile_lin = plan.full + t;
  const int ti = tile_lin / n_ntiles;
  const int* te = tiles + 4 + kTileInts * ti;
  const int first = te[3], cnt = te[4];
  const int o = tile_lin - first * n_ntiles;
  const int j = o / cnt;
  const int i = first + o % cnt;
  const int* td = tiles + 4 + kTileInts * i;
  const int seg = td[0], r0 = td[1], r1 = td[2];
  const int n0 = j * cols_per_tile;
  f32x16 acc[2][2];
  for (int p = 0; p < plan.s; ++p) {
    const float* src = partials + (size_t)(t * plan.s + p) * (kBM3 * kBN2) + (size_t)wn * (64 * 64);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const f32x16 v = *reinterpret_cast<const f32x16*>(src + ((mi * 2 + ni) * 64 + lane) * 16);
        acc[mi][ni] = p == 0 ? v : acc[mi][ni] + v;
      }
  }
  store_block64<MODE, HAS_BIAS>(acc, lds + wn * (32 * 64), lane, kh, l32, wn, r0, r1, n0, Nn, seg, bias, out);
}

// fp32 storage: one thread per output element, sequential fp32 FMA over K.
template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, int n_seg, int dense_rows,
    const float* __restrict__ W, const float* __restrict__ W3, const float* __restrict__ bias,
    float* __restrict__ out, int K, int Nn) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int rows = offsets ? offsets[n_seg] : dense_rows;
  if (i >= (size_t)rows * Nn) return;
  const int row = (int)(i / Nn), col = (int)(i % Nn);
  int seg = 0;
  if (offsets) {
    int lo = 0, hi = n_seg;                   // last seg with offsets[seg] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= row) lo = mid; else hi = mid;
    }
    seg = lo;
  }
  const float* a = A + (size_t)row * K;
  const float* w = W + (size_t)seg * Nn * K + (size_t)col * K;
  float acc = 0.f;
  for (int j = 0; j < K; ++j) acc = fmaf(a[j], w[j], acc);
  float v;
  if (MODE == MODE_SWIGLU_UP) {
    const float* w3 = W3 + (size_t)seg * Nn * K + (size_t)col * K;
    float acc3 = 0.f;
    for (int j = 0; j < K; ++j) acc3 = fmaf(a[j], w3[j], acc3);
    v = silu_f(acc) * acc3;
  } else {
    v = acc;
    if (HAS_BIAS) v += bias[(size_t)seg * Nn + col];
    if (MODE == MODE_GELU_UP) v = gelu_f(v);
  }
  out[i] = v;
}

int grouped_gemm_max_tiles(int max_rows, int n_seg) { return max_rows / 256 + n_seg; }
int grouped_gemm_max_small_tiles(int n_seg) { return 2 * n_seg; }
size_t grouped_gemm_partials_bytes() { return (size_t)kMaxSplitUnits * kBM2 * kBN2 * sizeof(float); }

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <int MODE, bool HAS_BIAS>
static void launch_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const int cols = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int n_ntiles = (g.Nn + cols - 1) / cols;
  const int grid = ((device_cus() + kXcds - 1) / kXcds) * kXcds;
  const uint16_t* a = (const uint16_t*)g.a;
  const uint16_t* w = (const uint16_t*)g.w;
  const uint16_t* w3 = (const uint16_t*)g.w3;
  const uint16_t* b = (const uint16_t*)g.bias;
  uint16_t* out = (uint16_t*)g.out;
  if (g.max_rows >= kBigTailMin) {   // otherwise no segment can hold a 256-row tile
    hipLaunchKernelGGL((grouped_gemm_256_kernel<MODE, HAS_BIAS>), dim3(grid), dim3(256), 0, s, a, g.tiles, w, w3,
                       b, out, g.partials, g.K, g.Nn, n_ntiles);
    hipLaunchKernelGGL((split_fixup_kernel<MODE, HAS_BIAS>), dim3(kMaxSplitUnits), dim3(256), 0, s, g.tiles,
                       (const float*)g.partials, b, out, g.Nn, n_ntiles, grid);
  }
  hipLaunchKernelGGL((grouped_gemm_64_kernel<MODE, HAS_BIAS>), dim3(grid), dim3(256), 0, s, a, g.tiles_small, w,
                     w3, b, out, g.partials, g.K, g.Nn, n_ntiles);
  hipLaunchKernelGGL((split_fixup64_kernel<MODE, HAS_BIAS>), dim3(kMaxSplitUnits), dim3(256), 0, s, g.tiles_small,
                     (const float*)g.partials, b, out, g.Nn, n_ntiles, grid);
}

template <int MODE, bool HAS_BIAS>
static void launch_f32(const GroupedGemmArgs& g, hipStream_t s) {
  const size_t n = (size_t)g.max_rows * g.Nn;
  hipLaunchKernelGGL((grouped_gemm_f32_kernel<MODE, HAS_BIAS>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                     0, s, (const float*)g.a, g.offsets, g.n_seg, g.max_rows, (const float*)g.w,
                     (const float*)g.w3, (const float*)g.bias, (float*)g.out, g.K, g.Nn);
}

hipError_t launch_grouped_gemm(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.max_rows <= 0) return hipSuccess;
  const bool hb = g.bias != nullptr;
  if (g.dtype == MOE_F32) {
    if (g.mode == MODE_SWIGLU_UP) launch_f32<MODE_SWIGLU_UP, false>(g, s);
    else if (g.mode == MODE_GELU_UP) hb ? launch_f32<MODE_GELU_UP, true>(g, s) : launch_f32<MODE_GELU_UP, false>(g, s);
    else hb ? launch_f32<MODE_DOWN, true>(g, s) : launch_f32<MODE_DOWN, false>(g, s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, g.offsets, g.n_seg, g.max_rows, g.tiles,
                     g.max_tiles, g.tiles_small, g.max_tiles_small);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (g.mode == MODE_SWIGLU_UP) launch_bf16<MODE_SWIGLU_UP, false>(g, s);
  else if (g.mode == MODE_GELU_UP) hb ? launch_bf16<MODE_GELU_UP, true>(g, s) : launch_bf16<MODE_GELU_UP, false>(g, s);
  else hb ? launch_bf16<MODE_DOWN, true>(g, s) : launch_bf16<MODE_DOWN, false>(g, s);
  return hipGetLastError();
}

}  // namespace moe
