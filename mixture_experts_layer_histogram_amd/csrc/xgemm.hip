// Products of the layer backward whose operands are K-major in memory.
//
//   NN (ragged rows):  out[r, n] = sum_k A[r, k] B_s[k, n] for the rows r of
//       segment s.  A is row-major [rows, K] in expert order; B_s is a weight
//       matrix in its stored layout, [K, N] with N contiguous, so
//       dH = dY W2_e (W2_e is [d, F]) and dX = [dA1 | dA3] [W1_e ; W3_e]
//       (W1_e, W3_e are [F, d]) need no transposed weight copies.
//   TN (ragged reduction): C_s[m, n] = sum over the rows r of segment s of
//       P[r, m] Q[r, n] in fp32: the weight gradients dW2_e = dY^T H,
//       dW1_e = dA1^T X, dW_router = dZ^T X.
//
// Both run the forward's 256 x 256 x 64 tile (8 wavefronts of 128 x 64, MFMA
// 32x32x16 bf16, two 64 KB LDS stages filled by direct-to-LDS buffer loads,
// one barrier per K step), plus a 128 x 128 TN tile for short segments.  What
// changes is how a K-major operand sits in LDS and reaches the MFMA:
//
// K-major stage: 64 K rows x 256 columns, 512 bytes per row; the 16-byte
// chunk c of row r sits in slot c ^ (4 (r & 3)).  A direct-to-LDS load moves
// two such rows (64 lanes x 16 bytes); the lane that fills slot s fetches
// source chunk s ^ (4 (r & 3)).
//
// Transposing fragment read: ds_read_b64_tr_b16 works on groups of 16 lanes;
// lane i of a group receives element i % 4 of the 8-byte blocks that lanes
// 4 j + i / 4 (j = 0..3) address.  So if lane i addresses row kb + i / 4,
// columns c0 + 4 (i % 4) .. + 3, it receives column c0 + i at rows kb .. kb + 3.
// The MFMA operand (column l % 32, K 8 (l / 32) .. + 7 for lane l) is two such
// reads: group G = l / 16 takes c0 = 16 (G & 1), kb = 8 (G >> 1) and kb + 4.
// Per half-wave the 16 (row, chunk) pairs of one read fall on 16 distinct
// 4-bank groups under the slot swizzle above.
#include <type_traits>

#include "gemm_tile.h"

namespace moe {

typedef __bf16 bf16x4t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4t lds_bf16x4;

__device__ __forceinline__ bf16x4t read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Lane constants of the transposing fragment reads of a K-major stage whose
// 128-column block for this wavefront starts at column `cblk` (a multiple of
// 128, so the swizzle can act on the chunk index within the block):
// element offset of fragment x (32 columns each) in sub-step kk, half h =
//   (16 kk + 4 h) * 256 + base + xo[x].
struct TrLane {
  int base;
  int xo[4];
};

__device__ __forceinline__ TrLane tr_lane(int lane, int cblk) {
  const int G = lane >> 4, i = lane & 15;
  const int row = 8 * (G >> 1) + (i >> 2);             // row within the sub-step
  const int chunk = 2 * (G & 1) + ((i & 3) >> 1);      // 16-byte chunk within the 32-column fragment
  const int sw = 4 * (i >> 2);                          // = 4 (row & 3)
  TrLane t;
  t.base = row * 256 + cblk + 4 * (i & 1);
#pragma unroll
  for (int x = 0; x < 4; ++x) t.xo[x] = ((4 * x + chunk) ^ sw) * 8;
  return t;
}

__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* st, const TrLane& t, int kk, int x) {
  const uint16_t* p = st + kk * 16 * 256 + t.base + t.xo[x];
  const bf16x4t lo = read_tr(p);
  const bf16x4t hi = read_tr(p + 4 * 256);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Arguments of the NN product.
struct NnParams {
  const uint16_t* A;        // [rows, K] in segment order
  const int32_t* tiles;     // 256-row tiles covering every row (kind 2)
  const uint16_t* B1;       // rows k < K1 of B_s: B1 + s * strideB + k * N
  const uint16_t* B2;       // rows k >= K1: B2 + s * strideB + (k - K1) * N (or null)
  long long strideB;
  int K, K1, N;
  int b_rows1, b_rows2;     // rows of B1 / B2 per segment that exist (beyond: zero)
  uint16_t* out;            // [rows, N]
  int n_ntiles;
};

// ---------------------------------------------------------------------------
// NN: persistent over the units of a 256-row tile list (expert-major, N-tile
// by N-tile over the expert's row tiles; each XCD a contiguous range), on 8
// wavefronts (two per SIMD) like the forward's 256-row tile: a 2 x 4 layout of
// 128 x 64 blocks (4 x 2 MFMA blocks, 128 accumulators per lane), so one
// wavefront of a SIMD issues MFMAs while the other waits.  Each wavefront
// loads 32 A rows and 8 K rows of B per step.
//
// Direct-to-LDS loads of a K-major operand: wavefront w fills K rows
// 8 w .. 8 w + 7 of the stage, two rows per instruction.  voff[u] is the byte
// offset of this lane's source chunk for instruction u at K row 0 of the
// operand (rows advance by `rowbytes`).
__device__ __forceinline__ void tr_dma_offsets8(int wave, int lane, int rowbytes, int col0, int (&voff)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int lr = 8 * wave + 2 * u + (lane >> 5);
    const int chunk = (lane & 31) ^ (4 * (lr & 3));
    voff[u] = lr * rowbytes + col0 * 2 + chunk * 16;
  }
}

// As tr_lane for a 64-column block at column cblk of the 256-column stage;
// the swizzle acts on the chunk index within the whole row (a 64-column block
// starts at chunk 8 wn, so it cannot be applied to the block's own index).
__device__ __forceinline__ TrLane tr_lane64(int lane, int cblk) {
  const int G = lane >> 4, i = lane & 15;
  const int row = 8 * (G >> 1) + (i >> 2);
  const int chunk = 2 * (G & 1) + ((i & 3) >> 1);
  const int sw = 4 * (i >> 2);
  TrLane t;
  t.base = row * 256 + 4 * (i & 1);
#pragma unroll
  for (int x = 0; x < 2; ++x) t.xo[x] = ((cblk / 8 + 4 * x + chunk) ^ sw) * 8;
  t.xo[2] = t.xo[3] = 0;
  return t;
}

__global__ __launch_bounds__(512, 1) void gemm_nn_kernel(NnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * kStageElems];
  const int G = gridDim.x;
  const int KT = p.K / kBK2;
  UnitPlan plan;
  plan.full = p.tiles[0] * p.n_ntiles;
  plan.rem = 0;
  plan.s = 1;
  const int U = plan.full;
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  const int span = (U + kXcds - 1) / kXcds;
  const int u0 = min(U, xcd * span), cnt = min(U, u0 + span) - u0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, kh = lane >> 5;
  const int rowbytes = p.K * 2, browbytes = p.N * 2;
  const int h = kh ^ swz8(l32);
  const int abase = (wm * 128 + l32) * kBK2;
  const TrLane tb = tr_lane64(lane, wn * 64);

  for (int it = q; it < cnt; it += per_xcd) {
    const Unit w = decode_unit(p.tiles, plan, u0 + it, p.n_ntiles, KT, kBN2);
    int voff[4], voffb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 32 * wave + 8 * u + (lane >> 3);
      voff[u] = row * rowbytes + (((lane & 7) ^ swz8(row)) * 16);
    }
    tr_dma_offsets8(wave, lane, browbytes, w.n0, voffb);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.A + (size_t)w.r0 * p.K, (uint32_t)(w.r1 - w.r0) * rowbytes);
    const __amdgpu_buffer_rsrc_t rb1 =
        make_rsrc(p.B1 + (size_t)w.seg * p.strideB, (uint32_t)p.b_rows1 * browbytes);
    const __amdgpu_buffer_rsrc_t rb2 =
        make_rsrc(p.B2 ? p.B2 + (size_t)w.seg * p.strideB : p.B1, p.B2 ? (uint32_t)p.b_rows2 * browbytes : 0u);

    auto issue = [&](uint16_t* st, int kt, int u) {
      dma16(ra, st + (32 * wave + 8 * u) * kBK2, voff[u], kt * kBK2 * 2);
      const int k0 = kt * kBK2;
      const bool second = k0 >= p.K1;
      const int kb = second ? k0 - p.K1 : k0;
      dma16(second ? rb2 : rb1, st + kStageElems + (8 * wave + 2 * u) * 256, voffb[u] + kb * browbytes, 0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    // live 32-row blocks of this wavefront (rows past the segment are zero and never stored)
    const int nv = __builtin_amdgcn_readfirstlane(min(4, max(0, (w.r1 - w.r0 - wm * 128 + 31) / 32)));
    auto step = [&](const uint16_t* __restrict__ st, uint16_t* __restrict__ nx, int kt, auto nv_t) {
      constexpr int NV = decltype(nv_t)::value;
      MOE_WAIT_VM0();
      __builtin_amdgcn_s_barrier();
      const bool more = kt + 1 < KT;
      bf16x8 fa[2][4], fb[2][2];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (x < NV) fa[0][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + ((h ^ (4 * (x & 1))) << 3));
#pragma unroll
      for (int x = 0; x < 2; ++x) fb[0][x] = frag_tr(st + kStageElems, tb, 0, x);
#pragma unroll
      for (int kk = 0; kk < kBK2 / 16; ++kk) {
        const int c = kk & 1;
        if (more && kk < 2) {
#pragma unroll
          for (int u = 2 * kk; u < 2 * kk + 2; ++u) issue(nx, kt + 1, u);
        }
        if (kk + 1 < kBK2 / 16) {
          const int k2 = 2 * (kk + 1);
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (x < NV)
              fa[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + ((h ^ (4 * (x & 1)) ^ k2) << 3));
#pragma unroll
          for (int x = 0; x < 2; ++x) fb[c ^ 1][x] = frag_tr(st + kStageElems, tb, kk + 1, x);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int mi = 0; mi < NV; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
      }
    };
    if (KT > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) issue(lds, 0, u);
    }
    auto loop = [&](auto nv_t) {
      for (int kt = 0; kt < KT; ++kt)
        step(lds + (kt & 1) * (2 * kStageElems), lds + ((kt + 1) & 1) * (2 * kStageElems), kt, nv_t);
    };
    switch (nv) {
      case 4: loop(std::integral_constant<int, 4>{}); break;
      case 3: loop(std::integral_constant<int, 3>{}); break;
      case 2: loop(std::integral_constant<int, 2>{}); break;
      case 1: loop(std::integral_constant<int, 1>{}); break;
      default: loop(std::integral_constant<int, 0>{}); break;
    }
    __syncthreads();
    // epilogue: this wavefront's 128 x 64 block through its 8 KB of LDS, 32 rows at a time
    float* ep = reinterpret_cast<float*>(lds) + wave * (32 * 64);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) ep[ep_at((r >> 2) * 8 + kh * 4 + (r & 3), ni * 32 + l32)] = acc[mi][ni][r];
      __builtin_amdgcn_wave_barrier();
      const int rbase = w.r0 + wm * 128 + mi * 32;
#pragma unroll 1
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const int row = rbase + rr, col = w.n0 + wn * 64 + c8;
        if (row < w.r1 && col < p.N) {
          float src[8];
#pragma unroll
          for (int q = 0; q < 2; ++q)
            *reinterpret_cast<float4*>(src + q * 4) = *reinterpret_cast<const float4*>(ep + ep_at(rr, c8 + q * 4));
          *reinterpret_cast<uint4*>(p.out + (size_t)row * p.N + col) = pack_bf16x8(src);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// TN: items (segment, M tile, N tile) in segment-major, M-tile-major order;
// segments longer than kTnShortRows rows run 256 x 256 tiles in
// gemm_tn_kernel, the others 128 x 128 tiles in gemm_tn_short_kernel.
struct TnParams {
  const uint16_t* P;        // [rows, ldp], columns pc0 .. pc0 + M
  const uint16_t* Q;        // [rows, ldq], columns 0 .. N
  const int32_t* offsets;   // segment row ranges, or null: one segment of dense_rows rows
  int dense_rows;
  int ldp, pc0, ldq;
  int M, N;
  float* C;                 // C_s = C + s * strideC, [M, N] row-major
  long long strideC;
  int tiles_m, tiles_n, units;
};

// Segments of at most this many rows go to gemm_tn_short_kernel.
constexpr int kTnShortRows = 256;

// One 256 x 256 TN tile on 8 wavefronts (2 x 4 layout of 128 x 64 blocks, as
// the NN kernel): P fragments through the 128-column lane map, Q fragments
// through the 64-column one; each wavefront loads 8 K rows of both operands.
__device__ __forceinline__ void tn_tile(const TnParams& p, uint16_t* lds, int s, int m0, int n0, int lo, int hi) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, kh = lane >> 5;
  const int pbytes = p.ldp * 2, qbytes = p.ldq * 2;
  int voffp[4], voffq[4];
  tr_dma_offsets8(wave, lane, pbytes, p.pc0 + m0, voffp);
  tr_dma_offsets8(wave, lane, qbytes, n0, voffq);
  const TrLane ta = tr_lane(lane, wm * 128), tb = tr_lane64(lane, wn * 64);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.P + (size_t)lo * p.ldp, (uint32_t)(hi - lo) * pbytes);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + (size_t)lo * p.ldq, (uint32_t)(hi - lo) * qbytes);

  auto issue = [&](uint16_t* st, int kt, int u) {
    const int r = kt * kBK2;
    dma16(rp, st + (8 * wave + 2 * u) * 256, voffp[u] + r * pbytes, 0);
    dma16(rq, st + kStageElems + (8 * wave + 2 * u) * 256, voffq[u] + r * qbytes, 0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int KT = (hi - lo + kBK2 - 1) / kBK2;
  auto step = [&](const uint16_t* __restrict__ st, uint16_t* __restrict__ nx, int kt) {
    MOE_WAIT_VM0();
    __builtin_amdgcn_s_barrier();
    const bool more = kt + 1 < KT;
    bf16x8 fa[2][4], fb[2][2];
#pragma unroll
    for (int x = 0; x < 4; ++x) fa[0][x] = frag_tr(st, ta, 0, x);
#pragma unroll
    for (int x = 0; x < 2; ++x) fb[0][x] = frag_tr(st + kStageElems, tb, 0, x);
#pragma unroll
    for (int kk = 0; kk < kBK2 / 16; ++kk) {
      const int c = kk & 1;
      if (more && kk < 2) {
#pragma unroll
        for (int u = 2 * kk; u < 2 * kk + 2; ++u) issue(nx, kt + 1, u);
      }
      if (kk + 1 < kBK2 / 16) {
#pragma unroll
        for (int x = 0; x < 4; ++x) fa[c ^ 1][x] = frag_tr(st, ta, kk + 1, x);
#pragma unroll
        for (int x = 0; x < 2; ++x) fb[c ^ 1][x] = frag_tr(st + kStageElems, tb, kk + 1, x);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  };
  if (KT > 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) issue(lds, 0, u);
  }
  for (int kt = 0; kt < KT; ++kt)
    step(lds + (kt & 1) * (2 * kStageElems), lds + ((kt + 1) & 1) * (2 * kStageElems), kt);
  __syncthreads();
  // epilogue: the wavefront's 128 x 64 fp32 block through its 8 KB of LDS, 32 rows at a time
  float* ep = reinterpret_cast<float*>(lds) + wave * (32 * 64);
  float* C = p.C + (size_t)s * p.strideC;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[ep_at((r >> 2) * 8 + kh * 4 + (r & 3), ni * 32 + l32)] = acc[mi][ni][r];
    __builtin_amdgcn_wave_barrier();
    const int rbase = m0 + wm * 128 + mi * 32;
#pragma unroll 1
    for (int pass = 0; pass < 8; ++pass) {
      const int rr = pass * 4 + (lane >> 4), c4 = (lane & 15) * 4;
      const int row = rbase + rr, col = n0 + wn * 64 + c4;
      if (row < p.M && col < p.N)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(ep + ep_at(rr, c4)),
                                    reinterpret_cast<f32x4*>(C + (size_t)row * p.N + col));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Persistent: grid = CUs rounded to a multiple of 8, a grid-stride loop over
// the items (segment-major, M-tile-major), skipping those of short segments.
// An item's work grows with its segment's length, so consecutive items are
// dealt round-robin over the XCDs (item % 8 = the workgroup's XCD): with
// contiguous XCD ranges a skewed routing left one XCD with three times the
// mean work.
__global__ __launch_bounds__(512, 1) void gemm_tn_kernel(TnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * kStageElems];
  for (int item = blockIdx.x; item < p.units; item += gridDim.x) {
    const int per_seg = p.tiles_m * p.tiles_n;
    const int s = item / per_seg;
    const int lo = __builtin_amdgcn_readfirstlane(p.offsets ? p.offsets[s] : 0);
    const int hi = __builtin_amdgcn_readfirstlane(p.offsets ? p.offsets[s + 1] : p.dense_rows);
    if (hi - lo <= kTnShortRows) continue;
    tn_tile(p, lds, s, ((item % per_seg) / p.tiles_n) * 256, (item % p.tiles_n) * 256, lo, hi);
    __syncthreads();   // the next tile's loads must not overtake this epilogue's LDS reads
  }
}

// ---------------------------------------------------------------------------
// TN for short segments (at most kTnShortRows rows: most experts of a skewed
// routing, and unused experts, whose gradient is zero).  There the product is
// bound by writing the fp32 gradient, so the tile is small and cheap to keep
// many of in flight: 128 x 128, 4 wavefronts of 64 x 64 (2 x 2 MFMA blocks),
// one 32 KB K-major stage per operand pair (64 K rows x 128 columns, 256 bytes
// per row, chunk c of row r in slot c ^ 4 (r & 3), the same swizzle as the
// 256-column stage: it only touches the low four bits of the chunk index), and
// the accumulators stored straight from registers (half a wavefront writes
// 128 contiguous bytes of one row) as nontemporal stores: the fp32 gradients
// are not read again here, and streaming them past the caches measured 1.5%
// faster.  Several workgroups share a CU, so one's
// stores overlap another's loads; each K step is load, barrier, 16 MFMAs.
__device__ __forceinline__ void tr_dma_offsets128(int wave, int lane, int rowbytes, int col0, int (&voff)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int lr = 16 * wave + 4 * u + (lane >> 4);
    const int chunk = (lane & 15) ^ (4 * (lr & 3));
    voff[u] = lr * rowbytes + col0 * 2 + chunk * 16;
  }
}

// As tr_lane for a 128-column stage; the wavefront's 64-column block starts
// at column cblk, and the swizzle is applied to the chunk index within the row.
__device__ __forceinline__ TrLane tr_lane128(int lane, int cblk) {
  const int G = lane >> 4, i = lane & 15;
  const int row = 8 * (G >> 1) + (i >> 2);
  const int chunk = 2 * (G & 1) + ((i & 3) >> 1);
  const int sw = 4 * (i >> 2);
  TrLane t;
  t.base = row * 128 + 4 * (i & 1);
#pragma unroll
  for (int x = 0; x < 2; ++x) t.xo[x] = ((cblk / 8 + 4 * x + chunk) ^ sw) * 8;
  t.xo[2] = t.xo[3] = 0;
  return t;
}

__device__ __forceinline__ bf16x8 frag_tr128(const uint16_t* st, const TrLane& t, int kk, int x) {
  const uint16_t* q = st + kk * 16 * 128 + t.base + t.xo[x];
  const bf16x4t lo = read_tr(q);
  const bf16x4t hi = read_tr(q + 4 * 128);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Persistent like gemm_tn_kernel over 128 x 128 items (p.tiles_m, p.tiles_n,
// p.units count those), skipping the items of long segments.
__global__ __launch_bounds__(256) void gemm_tn_short_kernel(TnParams p) {
  constexpr int kOp = 64 * 128;   // elements of one operand's stage
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kOp];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int pbytes = p.ldp * 2, qbytes = p.ldq * 2;
  const TrLane ta = tr_lane128(lane, wm * 64), tb = tr_lane128(lane, wn * 64);
  const int per_seg = p.tiles_m * p.tiles_n;
  for (int item = blockIdx.x; item < p.units; item += gridDim.x) {
    const int s = item / per_seg;
    const int lo = __builtin_amdgcn_readfirstlane(p.offsets ? p.offsets[s] : 0);
    const int hi = __builtin_amdgcn_readfirstlane(p.offsets ? p.offsets[s + 1] : p.dense_rows);
    const int rows = hi - lo;
    if (rows > kTnShortRows) continue;
    const int m0 = ((item % per_seg) / p.tiles_n) * 128, n0 = (item % p.tiles_n) * 128;
    int voffp[4], voffq[4];
    tr_dma_offsets128(wave, lane, pbytes, p.pc0 + m0, voffp);
    tr_dma_offsets128(wave, lane, qbytes, n0, voffq);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.P + (size_t)lo * p.ldp, (uint32_t)rows * pbytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + (size_t)lo * p.ldq, (uint32_t)rows * qbytes);
    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    for (int k0 = 0; k0 < rows; k0 += 64) {
      __syncthreads();   // every wavefront is done with the stage (and with the previous item)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dma16(rp, lds + (16 * wave + 4 * u) * 128, voffp[u] + k0 * pbytes, 0);
        dma16(rq, lds + kOp + (16 * wave + 4 * u) * 128, voffq[u] + k0 * qbytes, 0);
      }
      MOE_WAIT_VM0();
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          fa[x] = frag_tr128(lds, ta, kk, x);
          fb[x] = frag_tr128(lds + kOp, tb, kk, x);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
      }
    }
    float* C = p.C + (size_t)s * p.strideC;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int n = n0 + wn * 64 + ni * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
          if (m < p.M) __builtin_nontemporal_store(acc[mi][ni][r], C + (size_t)m * p.N + n);
        }
    }
  }
}

static int cus_rounded() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  return ((v + kXcds - 1) / kXcds) * kXcds;
}

hipError_t launch_gemm_nn(const void* A, const int32_t* offsets, int n_seg, int dense_rows, int max_rows,
                          int32_t* tiles, int max_tiles, int32_t* tiles_small, int max_tiles_small, const void* B1,
                          const void* B2, long long strideB, int K, int K1, int b_rows1, int b_rows2, int N, void* out,
                          hipStream_t s) {
  if (K % kBK2 != 0 || K1 % kBK2 != 0 || N % 8 != 0 || (B2 == nullptr && K1 < K)) return hipErrorInvalidValue;
  if ((size_t)b_rows1 * N * 2 >= 0x80000000ull || (size_t)b_rows2 * N * 2 >= 0x80000000ull ||
      (size_t)max_rows * K * 2 >= 0x80000000ull || max_tiles < max_rows / 256 + n_seg)
    return hipErrorInvalidValue;
  hipError_t e = launch_build_tiles(offsets, n_seg, dense_rows, tiles, max_tiles, tiles_small, max_tiles_small, 2, s);
  if (e != hipSuccess) return e;
  NnParams p;
  p.A = (const uint16_t*)A;
  p.tiles = tiles;
  p.B1 = (const uint16_t*)B1;
  p.B2 = (const uint16_t*)B2;
  p.strideB = strideB;
  p.K = K;
  p.K1 = K1;
  p.N = N;
  p.b_rows1 = b_rows1;
  p.b_rows2 = b_rows2;
  p.out = (uint16_t*)out;
  p.n_ntiles = (N + kBN2 - 1) / kBN2;
  hipLaunchKernelGGL(gemm_nn_kernel, dim3(cus_rounded()), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const void* P, int ldp, int pc0, const void* Q, int ldq, const int32_t* offsets, int n_seg,
                          int dense_rows, int max_seg_rows, int M, int N, float* C, long long strideC,
                          hipStream_t s) {
  if (n_seg == 0 || M == 0 || N == 0) return hipSuccess;
  if (ldp % 8 != 0 || pc0 % 8 != 0 || ldq % 8 != 0 || N % 8 != 0) return hipErrorInvalidValue;
  if ((size_t)max_seg_rows * ldp * 2 >= 0x80000000ull || (size_t)max_seg_rows * ldq * 2 >= 0x80000000ull)
    return hipErrorInvalidValue;
  TnParams p;
  p.P = (const uint16_t*)P;
  p.Q = (const uint16_t*)Q;
  p.offsets = offsets;
  p.dense_rows = dense_rows;
  p.ldp = ldp;
  p.pc0 = pc0;
  p.ldq = ldq;
  p.M = M;
  p.N = N;
  p.C = C;
  p.strideC = strideC;
  // dense: the one segment's length is known here; ragged: short segments can always occur
  const bool any_short = offsets != nullptr || dense_rows <= kTnShortRows;
  const bool any_long = offsets != nullptr ? max_seg_rows > kTnShortRows : dense_rows > kTnShortRows;
  const int grid = cus_rounded();
  if (any_short) {
    TnParams q = p;
    q.tiles_m = (M + 127) / 128;
    q.tiles_n = (N + 127) / 128;
    q.units = n_seg * q.tiles_m * q.tiles_n;
    hipLaunchKernelGGL(gemm_tn_short_kernel, dim3((unsigned)(4 * grid)), dim3(256), 0, s, q);
  }
  if (any_long) {
    p.tiles_m = (M + 255) / 256;
    p.tiles_n = (N + 255) / 256;
    p.units = n_seg * p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL(gemm_tn_kernel, dim3((unsigned)grid), dim3(512), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
