// Backward pass of the layer: gradients of the input, the router, the routed
// and shared experts, for an upstream gradient of the output and of the
// auxiliary loss.
//
// [L] "The load balance problem": the auxiliary loss is a second gradient
// signal into the router, and the selection bias moves after each training
// step (moe_bias_update); this file is the training step's backward half.
// The routing decisions (selection, capacity) are piecewise constant and
// taken as fixed; gradients flow through the gate weights, the kept slots'
// expert FFNs, the shared expert and the residual.
//
// Products run on the grouped GEMM of the forward pass (transposed weight
// copies make every operand contiguous along its reduction axis) and on the
// ragged-reduction kernel below for the weight gradients, whose reduction
// runs over each expert's rows.
#include "moe_internal.h"

#include <math.h>

namespace moe {

// ----------------------------------------------------------------- combine backward
// One wavefront per slot s = t k + j.  Kept slots: dg[t, j] = <dout_t, y_row>
// (fp32, lane-strided partial sums then a fixed xor tree) and dY_row =
// g[t, j] * dout_t.  Dropped slots: dg = 0.
template <typename T>
__global__ __launch_bounds__(256) void combine_backward_kernel(const T* __restrict__ dout, const T* __restrict__ y,
                                                               const int32_t* __restrict__ slot_pos,
                                                               const float* __restrict__ gates, int n_slots, int k,
                                                               int d, float* __restrict__ dg, T* __restrict__ dy) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  if (s >= n_slots) return;
  const int pos = slot_pos[s];
  if (pos < 0) {
    if (lane == 0) dg[s] = 0.f;
    return;
  }
  const int t = s / k;
  const float g = gates[s];
  const T* dr = dout + (size_t)t * d;
  const T* yr = y + (size_t)pos * d;
  T* dyr = dy + (size_t)pos * d;
  float acc = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float go = Store<T>::load(dr, c);
    acc = fmaf(go, Store<T>::load(yr, c), acc);
    Store<T>::store(dyr, c, g * go);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) dg[s] = acc;
}

// ----------------------------------------------------------------- transposes
// dst[b][c][col0 + r] = src[b][r][c] for a batch of [R, C] matrices (bf16),
// dst row stride ldd, through 64 x 64 LDS tiles.
//
// 16-byte form (R, C, ldd, col0 multiples of 8): each thread moves two
// 8-element row chunks in and two 8-element column chunks out, so global
// reads and writes are whole 128-byte lines per 8 lanes.  In LDS the 16-byte
// chunk c of tile row r sits at chunk c ^ ((r >> 3) & 7): the eight lanes
// that read one column at rows 8i + j then hit eight different chunks.
__global__ __launch_bounds__(256) void transpose8_kernel(const uint16_t* __restrict__ src, int R, int C,
                                                         uint16_t* __restrict__ dst, int ldd, int col0) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * 64];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t* s = src + (size_t)b * R * C;
  uint16_t* o = dst + (size_t)b * C * ldd;
#pragma unroll
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int rr = q >> 3, ch = q & 7;
    if (r0 + rr < R && c0 + ch * 8 < C)
      *reinterpret_cast<uint4*>(tile + rr * 64 + ((ch ^ ((rr >> 3) & 7)) << 3)) =
          *reinterpret_cast<const uint4*>(s + (size_t)(r0 + rr) * C + c0 + ch * 8);
  }
  __syncthreads();
#pragma unroll
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int cc = q >> 3, i = q & 7;      // output row c0 + cc, source rows 8 i .. 8 i + 7
    if (c0 + cc < C && r0 + 8 * i < R) {
      Vec8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v.e[j] = tile[(8 * i + j) * 64 + ((((cc >> 3) ^ i) & 7) << 3) + (cc & 7)];
      *reinterpret_cast<uint4*>(o + (size_t)(c0 + cc) * ldd + col0 + r0 + 8 * i) = v.u;
    }
  }
}

// Element form for other shapes.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src, int R, int C,
                                                        uint16_t* __restrict__ dst, int ldd, int col0) {
  __shared__ uint16_t tile[64][65];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t* s = src + (size_t)b * R * C;
  uint16_t* o = dst + (size_t)b * C * ldd;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    if (r0 + rr < R && c0 + cc < C) tile[rr][cc] = s[(size_t)(r0 + rr) * C + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (r0 + rr < R && c0 + cc < C) o[(size_t)(c0 + cc) * ldd + col0 + r0 + rr] = tile[rr][cc];
  }
}

// Zero columns [c0, c1) of a [rows, ld] bf16 matrix (K padding of a GEMM operand).
__global__ __launch_bounds__(256) void zero_cols_kernel(uint16_t* __restrict__ a, long long rows, int ld, int c0,
                                                        int c1) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int w = c1 - c0;
  if (w <= 0 || i >= rows * w) return;
  a[(size_t)(i / w) * ld + c0 + (int)(i % w)] = 0;
}

// ----------------------------------------------------------------- activation backward
// SwiGLU: from A1, A3 (pre-activations) and dH: H = SiLU(A1) A3, dA1 = dH A3
// SiLU'(A1), dA3 = dH SiLU(A1).  GELU: H = GELU(A), dA = dH GELU'(A).  fp32
// arithmetic, bf16 in and out.  dA rows are [dA1 | dA3] (row stride 2F) or
// [dA] (stride F).
__device__ __forceinline__ float sigmoid_f(float u) { return 1.0f / (1.0f + __expf(-u)); }

// One thread per 8 consecutive hidden units of a row (F a multiple of 8).
template <bool SWIGLU>
__global__ __launch_bounds__(256) void act_backward_kernel(const uint16_t* __restrict__ a1,
                                                           const uint16_t* __restrict__ a3,
                                                           const uint16_t* __restrict__ dh, long long rows, int F,
                                                           uint16_t* __restrict__ h, uint16_t* __restrict__ da) {
  const int F8 = F >> 3;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * F8) return;
  const long long r = i / F8;
  const int f = (int)(i % F8) * 8;
  const size_t e = (size_t)r * F + f;
  Vec8 u, g, hv, d1, d3;
  u.u = *reinterpret_cast<const uint4*>(a1 + e);
  g.u = *reinterpret_cast<const uint4*>(dh + e);
  if (SWIGLU) {
    Vec8 v;
    v.u = *reinterpret_cast<const uint4*>(a3 + e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float uu = bf16_to_f32(u.e[j]), gg = bf16_to_f32(g.e[j]), vv = bf16_to_f32(v.e[j]);
      const float sg = sigmoid_f(uu), si = uu * sg;
      hv.e[j] = f32_to_bf16(si * vv);
      d1.e[j] = f32_to_bf16(gg * vv * (sg * (1.0f + uu * (1.0f - sg))));
      d3.e[j] = f32_to_bf16(gg * si);
    }
    *reinterpret_cast<uint4*>(h + e) = hv.u;
    *reinterpret_cast<uint4*>(da + (size_t)r * 2 * F + f) = d1.u;
    *reinterpret_cast<uint4*>(da + (size_t)r * 2 * F + F + f) = d3.u;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float uu = bf16_to_f32(u.e[j]), gg = bf16_to_f32(g.e[j]);
      const float cdf = 0.5f * erfcf(-uu * 0.70710678118654752f);
      const float pdf = 0.39894228040143268f * __expf(-0.5f * uu * uu);
      hv.e[j] = f32_to_bf16(uu * cdf);
      d1.e[j] = f32_to_bf16(gg * (cdf + uu * pdf));
    }
    *reinterpret_cast<uint4*>(h + e) = hv.u;
    *reinterpret_cast<uint4*>(da + e) = d1.u;
  }
}

// ----------------------------------------------------------------- ragged-reduction GEMM
// Weight gradients: for each segment e (rows [offsets[e], offsets[e+1]), rows
// with perm < 0 skipped), C_e[m, n] = sum_r P[r, m] Q[r, n] in fp32, written
// to C + e * strideC (row stride ldc).  Q rows may be gathered token rows
// (Q row r = Qsrc[perm[r] / gk]).  P and Q are bf16 row-major with row
// strides ldp, ldq.
//
// 128 x 128 output tile per workgroup (4 wavefronts 2 x 2, each 64 x 64 =
// 2 x 2 MFMA 32x32x16 blocks).  K step = 32 rows: each thread loads two
// 16-byte pieces (rows r, r+1 of one 8-column chunk) per operand into
// registers, then writes them to LDS transposed ([column][row], rows padded
// to 40 elements) as 8 packed row pairs, so the MFMA fragments (8
// consecutive rows of one column) are single 16-byte LDS reads.  Two LDS
// stages; the next step's global loads are in flight during this step's
// MFMAs.
constexpr int kWgLd = 40;                       // LDS row length (elements) of the transposed tiles

template <bool GATHER_Q>
__global__ __launch_bounds__(256, 2) void wgrad_kernel(const uint16_t* __restrict__ P, int ldp,
                                                       const uint16_t* __restrict__ Q, int ldq,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ perm, int gk, int dense_rows,
                                                       int M, int N, float* __restrict__ C, int ldc,
                                                       long long strideC) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][128 * kWgLd];
  const int tiles_n = (N + 127) / 128;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int e = blockIdx.y;
  const int m0 = tm * 128, n0 = tn * 128;
  const int r_lo = offsets ? offsets[e] : 0;
  const int r_hi = offsets ? offsets[e + 1] : dense_rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, kh = lane >> 5;
  // loader: thread -> row pair rp (rows 2rp, 2rp+1 of the step), column chunk c (8 columns)
  const int rp = tid & 15, c = tid >> 4;

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  uint4 pv[2], qv[2];
  auto load = [&](int r0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + 2 * rp + h;
      bool ok = r < r_hi;
      int qrow = r;
      if (ok && perm != nullptr) {
        const int pr = perm[r];
        ok = pr >= 0;
        if (GATHER_Q) qrow = pr / gk;
      }
      const int mc = m0 + 8 * c, nc = n0 + 8 * c;
      pv[h] = (ok && mc < M) ? *reinterpret_cast<const uint4*>(P + (size_t)r * ldp + mc) : uint4{0, 0, 0, 0};
      qv[h] = (ok && nc < N) ? *reinterpret_cast<const uint4*>(Q + (size_t)qrow * ldq + nc) : uint4{0, 0, 0, 0};
    }
  };
  auto store = [&](int st) {
    uint32_t* lp = reinterpret_cast<uint32_t*>(lds[st][0]);
    uint32_t* lq = reinterpret_cast<uint32_t*>(lds[st][1]);
    const uint16_t* p0 = reinterpret_cast<const uint16_t*>(&pv[0]);
    const uint16_t* p1 = reinterpret_cast<const uint16_t*>(&pv[1]);
    const uint16_t* q0 = reinterpret_cast<const uint16_t*>(&qv[0]);
    const uint16_t* q1 = reinterpret_cast<const uint16_t*>(&qv[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lp[((8 * c + i) * kWgLd) / 2 + rp] = (uint32_t)p0[i] | ((uint32_t)p1[i] << 16);
      lq[((8 * c + i) * kWgLd) / 2 + rp] = (uint32_t)q0[i] | ((uint32_t)q1[i] << 16);
    }
  };

  const int steps = (r_hi - r_lo + 31) / 32;
  if (steps > 0) {
    load(r_lo);
    store(0);
    __syncthreads();
  }
  for (int s = 0; s < steps; ++s) {
    const int st = s & 1;
    if (s + 1 < steps) load(r_lo + 32 * (s + 1));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        fa[x] = *reinterpret_cast<const bf16x8*>(&lds[st][0][(wm * 64 + 32 * x + l32) * kWgLd + 16 * kk + 8 * kh]);
        fb[x] = *reinterpret_cast<const bf16x8*>(&lds[st][1][(wn * 64 + 32 * x + l32) * kWgLd + 16 * kk + 8 * kh]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    if (s + 1 < steps) store(st ^ 1);
    __syncthreads();
  }
  float* out = C + (size_t)e * strideC;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int n = n0 + wn * 64 + ni * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (m < M && n < N) out[(size_t)m * ldc + n] = acc[mi][ni][r];
      }
    }
}

// ----------------------------------------------------------------- column sums per segment
// Bias gradients: out[e][c] = sum over the segment's valid rows of a[r][col0 + c]
// (fp32).  Block = (512-column group, segment): each thread owns 8 adjacent
// columns (one 16-byte load per row), the 8 waves take every 8th row, and the
// wave partials are added in wave order, so the result is deterministic.
// Needs lda, col0 and ncols multiples of 8 (the scalar kernel below otherwise).
__global__ __launch_bounds__(512) void segment_colsum8_kernel(const uint16_t* __restrict__ a, int lda, int col0,
                                                              int ncols, const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ perm, int dense_rows,
                                                              float* __restrict__ out) {
  __shared__ float red[8][512];
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c0 = blockIdx.x * 512 + lane * 8;
  const int lo = offsets ? offsets[e] : 0, hi = offsets ? offsets[e + 1] : dense_rows;
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.f;
  if (c0 < ncols) {
    for (int r = lo + wave; r < hi; r += 8) {
      if (perm != nullptr && perm[r] < 0) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(a + (size_t)r * lda + col0 + c0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += __uint_as_float(w[i] << 16);
        s[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = s[i];
  __syncthreads();
  const int c = blockIdx.x * 512 + threadIdx.x;
  if (c < ncols) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) t += red[w][threadIdx.x];
    out[(size_t)e * ncols + c] = t;
  }
}

// Scalar form for unaligned strides: one thread per (segment, column), rows in order.
__global__ __launch_bounds__(256) void segment_colsum_kernel(const uint16_t* __restrict__ a, int lda, int col0,
                                                             int ncols, const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ perm, int dense_rows,
                                                             int n_seg, float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n_seg * ncols) return;
  const int e = (int)(i / ncols), cc = (int)(i % ncols);
  const int lo = offsets ? offsets[e] : 0, hi = offsets ? offsets[e + 1] : dense_rows;
  float s = 0.f;
  for (int r = lo; r < hi; ++r)
    if (perm == nullptr || perm[r] >= 0) s += bf16_to_f32(a[(size_t)r * lda + col0 + cc]);
  out[i] = s;
}

// Column sums of an fp32 [rows, cols] matrix in two deterministic passes:
// block b adds rows [256 b, 256 b + 256) of every column (wave w takes the
// rows = w mod 4; the four wave sums are added in order) into part[b][c];
// the second pass adds the chunk sums in ascending chunk order.
constexpr int kColsumChunk = 256;

__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ a, int rows, int cols,
                                                          float* __restrict__ part) {
  __shared__ float red[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * kColsumChunk, r1 = min(rows, r0 + kColsumChunk);
  for (int cb = 0; cb < cols; cb += 64) {
    const int c = cb + lane;
    float s = 0.f;
    if (c < cols) {
#pragma unroll 8
      for (int r = r0 + wave; r < r1; r += 4) s += a[(size_t)r * cols + c];
    }
    red[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && c < cols)
      part[(size_t)blockIdx.x * cols + c] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int nchunk, int cols,
                                                           float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
#pragma unroll 8
  for (int i = 0; i < nchunk; ++i) s += part[(size_t)i * cols + c];
  out[c] = s;
}

// ----------------------------------------------------------------- router backward
// One wavefront per token: p = softmax(z) (fp32, max subtracted); dz from the
// gate gradients by the gate rule, plus the aux-loss term d_aux E f_e / N
// through the softmax.  Writes dz (fp32 [N, E]) and a bf16 copy with row
// stride ldz (K-padded for the GEMM that forms dx).
__global__ __launch_bounds__(256) void router_backward_kernel(const float* __restrict__ z,
                                                              const int32_t* __restrict__ idx,
                                                              const float* __restrict__ gates,
                                                              const float* __restrict__ dg,
                                                              const int32_t* __restrict__ counts, float d_aux,
                                                              int N, int E, int k, int rule,
                                                              float* __restrict__ dz, uint16_t* __restrict__ dz16,
                                                              int ldz) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;
  const float* zr = z + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, zr[e]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float sum = 0.f;
  for (int e = lane; e < E; e += 64) sum += __expf(zr[e] - m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  // <g, dg> and sum of p over the selected experts (rule B)
  float gdg = 0.f, psel = 0.f;
  for (int j = 0; j < k; ++j) {
    gdg += gates[(size_t)t * k + j] * dg[(size_t)t * k + j];
    psel += __expf(zr[idx[(size_t)t * k + j]] - m) / sum;
  }
  const float aux_c = d_aux * (float)E / ((float)N * (float)N * (float)k);   // d_aux E f_e / N = aux_c * counts_e
  // dp (rules B, C and the aux term) and <p, dp>
  float pdp = 0.f;
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(zr[e] - m) / sum;
    float dp = counts ? aux_c * (float)counts[e] : 0.f;
    for (int j = 0; j < k; ++j) {
      if (idx[(size_t)t * k + j] != e) continue;
      const float gd = dg[(size_t)t * k + j];
      if (rule == MOE_GATE_SOFTMAX_RENORM) dp += (gd - gdg) / psel;
      else if (rule == MOE_GATE_SWITCH_TOP1) dp += gd;
    }
    pdp += p * dp;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pdp += __shfl_xor(pdp, off);
  for (int e = lane; e < ldz; e += 64) {
    float v = 0.f;
    if (e < E) {
      const float p = __expf(zr[e] - m) / sum;
      float dp = counts ? aux_c * (float)counts[e] : 0.f;
      float da = 0.f;
      for (int j = 0; j < k; ++j) {
        if (idx[(size_t)t * k + j] != e) continue;
        const float gd = dg[(size_t)t * k + j];
        if (rule == MOE_GATE_SOFTMAX_RENORM) dp += (gd - gdg) / psel;
        else if (rule == MOE_GATE_SWITCH_TOP1) dp += gd;
        else da += gates[(size_t)t * k + j] * (gd - gdg);   // rule A: softmax over the selected logits
      }
      v = p * (dp - pdp) + da;
      dz[(size_t)t * E + e] = v;
    }
    if (dz16) dz16[(size_t)t * ldz + e] = f32_to_bf16(v);
  }
}

// ----------------------------------------------------------------- dx
// dx[t] = [dout_t] + sum_j dX[slot_pos[t k + j]] + [dxs_t] + [dxr_t], fp32 accumulation in a
// fixed order, rounded once to the storage type.  One wavefront per token.
template <typename T>
__global__ __launch_bounds__(256) void dx_gather_kernel(const T* __restrict__ dout, const T* __restrict__ dX,
                                                        const int32_t* __restrict__ slot_pos,
                                                        const T* __restrict__ dxs, const T* __restrict__ dxr,
                                                        int N, int k, int d, T* __restrict__ dx) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;
  for (int c = lane; c < d; c += 64) {
    float a = dout ? Store<T>::load(dout, (size_t)t * d + c) : 0.f;
    for (int j = 0; j < k; ++j) {
      const int pos = slot_pos[(size_t)t * k + j];
      if (pos >= 0) a += Store<T>::load(dX, (size_t)pos * d + c);
    }
    if (dxs) a += Store<T>::load(dxs, (size_t)t * d + c);
    if (dxr) a += Store<T>::load(dxr, (size_t)t * d + c);
    Store<T>::store(dx, (size_t)t * d + c, a);
  }
}

// ----------------------------------------------------------------- launches
hipError_t launch_combine_backward(const moe_config& c, const void* dout, const void* y, const int32_t* slot_pos,
                                   const float* gates, float* dg, void* dy, hipStream_t s) {
  const int n_slots = (int)(c.n_tokens * c.top_k);
  if (n_slots == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_backward_kernel<uint16_t>, dim3((n_slots + 3) / 4), dim3(256), 0, s,
                     (const uint16_t*)dout, (const uint16_t*)y, slot_pos, gates, n_slots, c.top_k, c.d_model, dg,
                     (uint16_t*)dy);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int batch, int R, int C, void* dst, int ldd, int col0, hipStream_t s) {
  if (batch == 0 || R == 0 || C == 0) return hipSuccess;
  const bool vec = R % 8 == 0 && C % 8 == 0 && ldd % 8 == 0 && col0 % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  hipLaunchKernelGGL(vec ? transpose8_kernel : transpose_kernel, dim3((C + 63) / 64, (R + 63) / 64, batch), dim3(256), 0, s,
                     (const uint16_t*)src, R, C, (uint16_t*)dst, ldd, col0);
  return hipGetLastError();
}

hipError_t launch_zero_cols(void* a, long long rows, int ld, int c0, int c1, hipStream_t s) {
  const long long n = rows * (long long)(c1 - c0);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint16_t*)a, rows, ld,
                     c0, c1);
  return hipGetLastError();
}

hipError_t launch_act_backward(bool swiglu, const void* a1, const void* a3, const void* dh, long long rows, int F,
                               void* h, void* da, hipStream_t s) {
  if (F % 8 != 0) return hipErrorInvalidValue;
  const long long n = rows * (F / 8);
  if (n == 0) return hipSuccess;
  const dim3 g((unsigned)((n + 255) / 256));
  if (swiglu)
    hipLaunchKernelGGL(act_backward_kernel<true>, g, dim3(256), 0, s, (const uint16_t*)a1, (const uint16_t*)a3,
                       (const uint16_t*)dh, rows, F, (uint16_t*)h, (uint16_t*)da);
  else
    hipLaunchKernelGGL(act_backward_kernel<false>, g, dim3(256), 0, s, (const uint16_t*)a1, nullptr,
                       (const uint16_t*)dh, rows, F, (uint16_t*)h, (uint16_t*)da);
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* P, int ldp, const void* Q, int ldq, bool gather_q, const int32_t* offsets,
                        const int32_t* perm, int gk, int dense_rows, int n_seg, int M, int N, float* C, int ldc,
                        long long strideC, hipStream_t s) {
  if (n_seg == 0 || M == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)(((M + 127) / 128) * ((N + 127) / 128)), (unsigned)n_seg);
  if (gather_q)
    hipLaunchKernelGGL(wgrad_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)P, ldp, (const uint16_t*)Q, ldq,
                       offsets, perm, gk, dense_rows, M, N, C, ldc, strideC);
  else
    hipLaunchKernelGGL(wgrad_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)P, ldp, (const uint16_t*)Q,
                       ldq, offsets, perm, gk, dense_rows, M, N, C, ldc, strideC);
  return hipGetLastError();
}

hipError_t launch_segment_colsum(const void* a, int lda, int col0, int ncols, const int32_t* offsets,
                                 const int32_t* perm, int dense_rows, int n_seg, float* out, hipStream_t s) {
  const long long n = (long long)n_seg * ncols;
  if (n == 0) return hipSuccess;
  if (lda % 8 == 0 && col0 % 8 == 0 && ncols % 8 == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0) {
    hipLaunchKernelGGL(segment_colsum8_kernel, dim3((unsigned)((ncols + 511) / 512), (unsigned)n_seg), dim3(512), 0,
                       s, (const uint16_t*)a, lda, col0, ncols, offsets, perm, dense_rows, out);
  } else {
    hipLaunchKernelGGL(segment_colsum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)a, lda, col0, ncols, offsets, perm, dense_rows, n_seg, out);
  }
  return hipGetLastError();
}

size_t colsum_part_floats(int rows, int cols) {
  return (size_t)((rows + kColsumChunk - 1) / kColsumChunk) * (size_t)cols;
}

hipError_t launch_colsum_f32(const float* a, int rows, int cols, float* part, float* out, hipStream_t s) {
  if (cols == 0) return hipSuccess;
  const int nchunk = (rows + kColsumChunk - 1) / kColsumChunk;
  if (nchunk > 0)
    hipLaunchKernelGGL(colsum_part_kernel, dim3(nchunk), dim3(256), 0, s, a, rows, cols, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 255) / 256), dim3(256), 0, s, part, nchunk, cols, out);
  return hipGetLastError();
}

hipError_t launch_router_backward(const moe_config& c, const float* z, const int32_t* idx, const float* gates,
                                  const float* dg, const int32_t* counts, float d_aux, float* dz, void* dz16,
                                  int ldz, hipStream_t s) {
  const int N = (int)c.n_tokens;
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(router_backward_kernel, dim3((N + 3) / 4), dim3(256), 0, s, z, idx, gates, dg, counts, d_aux,
                     N, c.n_experts, c.top_k, c.gate_rule, dz, (uint16_t*)dz16, ldz);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const moe_config& c, const void* dout, const void* dX, const int32_t* slot_pos,
                            const void* dxs, const void* dxr, void* dx, hipStream_t s) {
  const int N = (int)c.n_tokens;
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(dx_gather_kernel<uint16_t>, dim3((N + 3) / 4), dim3(256), 0, s, (const uint16_t*)dout,
                     (const uint16_t*)dX, slot_pos, (const uint16_t*)dxs, (const uint16_t*)dxr, N, c.top_k,
                     c.d_model, (uint16_t*)dx);
  return hipGetLastError();
}

}  // namespace moe
