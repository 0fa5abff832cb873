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
// Products with the weights in their stored layout and the weight gradients
// (reductions over each expert's rows) run on the K-major tile kernels of
// xgemm.hip; the pre-activations are recomputed on the forward's grouped GEMM.
// The element kernels here: combine backward, activation backward, router
// backward, bias and logit-bias column sums, the expert-order row gather, and
// the final scatter of dx.
#include "moe_internal.h"

#include <math.h>

#include <algorithm>

namespace moe {

// ----------------------------------------------------------------- combine backward
// One wavefront per slot s = t k + j.  Kept slots: dg[t, j] = <dout_t, y_row>
// (fp32, lane-strided partial sums then a fixed xor tree) and dY_row =
// g[t, j] * dout_t.  Dropped slots: dg = 0.  16-byte lanes (d a multiple of 8).
__global__ __launch_bounds__(256) void combine_backward_kernel(const uint16_t* __restrict__ dout,
                                                               const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ slot_pos,
                                                               const float* __restrict__ gates, int n_slots, int k,
                                                               int d, float* __restrict__ dg,
                                                               uint16_t* __restrict__ dy) {
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
  const uint4* dr = reinterpret_cast<const uint4*>(dout + (size_t)t * d);
  const uint4* yr = reinterpret_cast<const uint4*>(y + (size_t)pos * d);
  uint4* dyr = reinterpret_cast<uint4*>(dy + (size_t)pos * d);
  float acc = 0.f;
  for (int c = lane; c < d / 8; c += 64) {
    Vec8 go, yv, o;
    go.u = dr[c];
    yv.u = yr[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gv = bf16_to_f32(go.e[e]);
      acc = fmaf(gv, bf16_to_f32(yv.e[e]), acc);
      o.e[e] = f32_to_bf16(g * gv);
    }
    dyr[c] = o.u;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) dg[s] = acc;
}

// ----------------------------------------------------------------- expert-order rows
// For the expert-order rows r < offsets[n_seg]: xg[r] = x[perm[r] / k] (the
// token row of the slot), and for padding rows of the [E, C] layout (perm < 0)
// xg[r] = 0 and dy[r] = 0, so every product over expert-order rows sees zeros
// there.  One wavefront per row, 16-byte lanes (d a multiple of 8).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets, int n_seg, int k,
                                                          int d, uint16_t* __restrict__ xg, uint16_t* __restrict__ dy) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + wave;
  if (r >= offsets[n_seg]) return;
  const int pr = perm[r];
  uint4* dst = reinterpret_cast<uint4*>(xg + (size_t)r * d);
  const int n8 = d / 8;
  if (pr >= 0) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)(pr / k) * d);
    for (int c = lane; c < n8; c += 64) dst[c] = src[c];
  } else {
    uint4* dyr = reinterpret_cast<uint4*>(dy + (size_t)r * d);
    for (int c = lane; c < n8; c += 64) {
      dst[c] = uint4{0, 0, 0, 0};
      dyr[c] = uint4{0, 0, 0, 0};
    }
  }
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
// fixed order, rounded once to bf16.  One wavefront per token, 16-byte lanes.
__device__ __forceinline__ void add8(float (&a)[8], const uint4& v) {
  Vec8 x;
  x.u = v;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] += bf16_to_f32(x.e[e]);
}

template <int KM>
__global__ __launch_bounds__(256) void dx_gather_kernel(const uint16_t* __restrict__ dout,
                                                        const uint16_t* __restrict__ dX,
                                                        const int32_t* __restrict__ slot_pos,
                                                        const uint16_t* __restrict__ dxs,
                                                        const uint16_t* __restrict__ dxr, int N, int k, int d,
                                                        uint16_t* __restrict__ dx) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;
  const size_t row = (size_t)t * d;
  int pos[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
  for (int c = lane; c < d / 8; c += 64) {
    // every slot's row loaded before the first is added (no branch around the loads:
    // dropped slots and slots past k read row 0 and are not added)
    uint4 r[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) r[j] = reinterpret_cast<const uint4*>(dX + (size_t)(pos[j] >= 0 ? pos[j] : 0) * d)[c];
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (dout) add8(a, reinterpret_cast<const uint4*>(dout + row)[c]);
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (pos[j] >= 0) add8(a, r[j]);
    if (dxs) add8(a, reinterpret_cast<const uint4*>(dxs + row)[c]);
    if (dxr) add8(a, reinterpret_cast<const uint4*>(dxr + row)[c]);
    Vec8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.e[e] = f32_to_bf16(a[e]);
    reinterpret_cast<uint4*>(dx + row)[c] = o.u;
  }
}

// Zero fill of an fp32 array (a kernel rather than a memset node, so callers
// may capture it in a graph).
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ----------------------------------------------------------------- launches
hipError_t launch_combine_backward(const moe_config& c, const void* dout, const void* y, const int32_t* slot_pos,
                                   const float* gates, float* dg, void* dy, hipStream_t s) {
  const int n_slots = (int)(c.n_tokens * c.top_k);
  if (n_slots == 0) return hipSuccess;
  if (c.d_model % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_backward_kernel, dim3((n_slots + 3) / 4), dim3(256), 0, s,
                     (const uint16_t*)dout, (const uint16_t*)y, slot_pos, gates, n_slots, c.top_k, c.d_model, dg,
                     (uint16_t*)dy);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm, const int32_t* offsets, int n_seg, int k, int d,
                              long long max_rows, void* xg, void* dy, hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((max_rows + 3) / 4)), dim3(256), 0, s, (const uint16_t*)x,
                     perm, offsets, n_seg, k, d, (uint16_t*)xg, (uint16_t*)dy);
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
  if (c.d_model % 8 != 0) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((N + 3) / 4), dim3(256), 0, s, (const uint16_t*)dout, (const uint16_t*)dX,
                       slot_pos, (const uint16_t*)dxs, (const uint16_t*)dxr, N, c.top_k, c.d_model, (uint16_t*)dx);
  };
  if (c.top_k <= 2) go(dx_gather_kernel<2>);
  else if (c.top_k <= 4) go(dx_gather_kernel<4>);
  else if (c.top_k <= 8) go(dx_gather_kernel<8>);
  else go(dx_gather_kernel<kMaxTopK>);
  return hipGetLastError();
}

}  // namespace moe
