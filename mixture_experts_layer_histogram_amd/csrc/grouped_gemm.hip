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

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;

// tiles[0] = tile count; tile i at tiles[4 + 4 i] = (segment, row_begin, row_end, 0).
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets, int n_seg,
                                                          int dense_rows, int block_m,
                                                          int32_t* __restrict__ tiles, int max_tiles) {
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int lo = 0, hi = 0, nt = 0;
  if (tid < n_seg) {
    lo = offsets ? offsets[tid] : 0;
    hi = offsets ? offsets[tid + 1] : dense_rows;
    nt = (hi - lo + block_m - 1) / block_m;
  }
  int incl = nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - nt;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  for (int i = 0; i < nt; ++i) {
    const int id = base + i;
    if (id >= max_tiles) break;
    int4 t;
    t.x = tid;
    t.y = lo + i * block_m;
    t.z = min(hi, lo + (i + 1) * block_m);
    t.w = 0;
    reinterpret_cast<int4*>(tiles + 4)[id] = t;
  }
  if (tid == 0) {
    const int tot = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    tiles[0] = min(tot, max_tiles);
  }
}

template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ tiles, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    int K, int Nn) {
  __shared__ uint16_t As[2][kBM * kLDK];
  __shared__ uint16_t Bs[2][kBN * kLDK];

  const int tile = blockIdx.x;
  if (tile >= tiles[0]) return;
  const int4 td = reinterpret_cast<const int4*>(tiles + 4)[tile];
  const int seg = td.x, r0 = td.y, r1 = td.z;
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN / 2 : kBN;
  const int n0 = blockIdx.y * cols_per_tile;

  const int tid = threadIdx.x;
  const int lr = tid >> 3, lc = tid & 7;      // global->LDS copy: row lr + 32 i, 16-byte chunk lc
  const size_t wstride = (size_t)Nn * K;      // elements per expert weight matrix
  const uint16_t* a_ptr0;
  const uint16_t* a_ptr1;
  const uint16_t* a_ptr2;
  const uint16_t* a_ptr3;
  const uint16_t* b_ptr0;
  const uint16_t* b_ptr1;
  const uint16_t* b_ptr2;
  const uint16_t* b_ptr3;
#define MOE_ROW_PTRS(i)                                                               \
  {                                                                                   \
    const int row = lr + 32 * i;                                                      \
    int ar = r0 + row;                                                                \
    if (ar > r1 - 1) ar = r1 - 1;                                                     \
    a_ptr##i = A + (size_t)ar * K + lc * 8;                                           \
    const uint16_t* wb = W;                                                           \
    int n = n0 + row;                                                                 \
    if (MODE == MODE_SWIGLU_UP && row >= 64) { n = n0 + row - 64; wb = W3; }          \
    if (n > Nn - 1) n = Nn - 1;                                                       \
    b_ptr##i = wb + (size_t)seg * wstride + (size_t)n * K + lc * 8;                   \
  }
  MOE_ROW_PTRS(0) MOE_ROW_PTRS(1) MOE_ROW_PTRS(2) MOE_ROW_PTRS(3)
#undef MOE_ROW_PTRS

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int brow0 = MODE == MODE_SWIGLU_UP ? wn * 32 + l32 : wn * 64 + l32;
  const int brow1 = MODE == MODE_SWIGLU_UP ? 64 + wn * 32 + l32 : wn * 64 + 32 + l32;

  f32x16 acc00, acc01, acc10, acc11;
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc00[r] = 0.f; acc01[r] = 0.f; acc10[r] = 0.f; acc11[r] = 0.f; }

  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define MOE_GLOAD(kt)                                                                 \
  {                                                                                   \
    const size_t ko = (size_t)(kt) * kBK;                                             \
    ra0 = *reinterpret_cast<const uint4*>(a_ptr0 + ko);                               \
    ra1 = *reinterpret_cast<const uint4*>(a_ptr1 + ko);                               \
    ra2 = *reinterpret_cast<const uint4*>(a_ptr2 + ko);                               \
    ra3 = *reinterpret_cast<const uint4*>(a_ptr3 + ko);                               \
    rb0 = *reinterpret_cast<const uint4*>(b_ptr0 + ko);                               \
    rb1 = *reinterpret_cast<const uint4*>(b_ptr1 + ko);                               \
    rb2 = *reinterpret_cast<const uint4*>(b_ptr2 + ko);                               \
    rb3 = *reinterpret_cast<const uint4*>(b_ptr3 + ko);                               \
  }
#define MOE_LSTORE(buf)                                                               \
  {                                                                                   \
    uint16_t* as = &As[buf][lr * kLDK + lc * 8];                                      \
    uint16_t* bs = &Bs[buf][lr * kLDK + lc * 8];                                      \
    *reinterpret_cast<uint4*>(as) = ra0;                                              \
    *reinterpret_cast<uint4*>(as + 32 * kLDK) = ra1;                                  \
    *reinterpret_cast<uint4*>(as + 64 * kLDK) = ra2;                                  \
    *reinterpret_cast<uint4*>(as + 96 * kLDK) = ra3;                                  \
    *reinterpret_cast<uint4*>(bs) = rb0;                                              \
    *reinterpret_cast<uint4*>(bs + 32 * kLDK) = rb1;                                  \
    *reinterpret_cast<uint4*>(bs + 64 * kLDK) = rb2;                                  \
    *reinterpret_cast<uint4*>(bs + 96 * kLDK) = rb3;                                  \
  }

  const int KT = K / kBK;
  MOE_GLOAD(0)
  MOE_LSTORE(0)
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) MOE_GLOAD(kt + 1)
    const uint16_t* as = &As[cur][(wm * 64 + l32) * kLDK + kh * 8];
    const uint16_t* bs0 = &Bs[cur][brow0 * kLDK + kh * 8];
    const uint16_t* bs1 = &Bs[cur][brow1 * kLDK + kh * 8];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(as + kk * 16);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(as + 32 * kLDK + kk * 16);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bs0 + kk * 16);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bs1 + kk * 16);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc11, 0, 0, 0);
    }
    if (more) MOE_LSTORE(cur ^ 1)
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_LSTORE

  // epilogue
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const f32x16& c0 = mi == 0 ? acc00 : acc10;
    const f32x16& c1 = mi == 0 ? acc01 : acc11;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + wm * 64 + mi * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
      if (row >= r1) continue;
      if (MODE == MODE_SWIGLU_UP) {
        const int col = n0 + wn * 32 + l32;
        if (col < Nn) {
          const float h = silu_f(c0[r]) * c1[r];
          out[(size_t)row * Nn + col] = f32_to_bf16(h);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + wn * 64 + ni * 32 + l32;
          if (col >= Nn) continue;
          float v = ni == 0 ? c0[r] : c1[r];
          if (HAS_BIAS) v += bf16_to_f32(bias[(size_t)seg * Nn + col]);
          if (MODE == MODE_GELU_UP) v = gelu_f(v);
          out[(size_t)row * Nn + col] = f32_to_bf16(v);
        }
      }
    }
  }
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

int grouped_gemm_max_tiles(int max_rows, int n_seg, int block_m) {
  return (max_rows + block_m - 1) / block_m + n_seg;
}

template <int MODE, bool HAS_BIAS>
static void launch_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const int cols = MODE == MODE_SWIGLU_UP ? kBN / 2 : kBN;
  dim3 grid(g.max_tiles, (g.Nn + cols - 1) / cols);
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<MODE, HAS_BIAS>), grid, dim3(256), 0, s,
                     (const uint16_t*)g.a, g.tiles, (const uint16_t*)g.w, (const uint16_t*)g.w3,
                     (const uint16_t*)g.bias, (uint16_t*)g.out, g.K, g.Nn);
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
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, g.offsets, g.n_seg, g.max_rows,
                     g.block_m, g.tiles, g.max_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (g.mode == MODE_SWIGLU_UP) launch_bf16<MODE_SWIGLU_UP, false>(g, s);
  else if (g.mode == MODE_GELU_UP) hb ? launch_bf16<MODE_GELU_UP, true>(g, s) : launch_bf16<MODE_GELU_UP, false>(g, s);
  else hb ? launch_bf16<MODE_DOWN, true>(g, s) : launch_bf16<MODE_DOWN, false>(g, s);
  return hipGetLastError();
}

int gemm_block_m(const moe_config&) { return kBM; }

}  // namespace moe
