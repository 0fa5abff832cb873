// Router: logits z = x W_r^T (+ logit bias), then per-token top-k selection and
// gate weights.
//
// [L] "Mixture of Experts (MoE)" lesson, "Build it / Step 1: the router": a
// token's score for expert e is its dot product with router row e; the experts
// are ranked by (score + bias) and the k best kept; the gates are a softmax
// over the chosen experts' raw scores.  [L] "The load balance problem"
// (DeepSeek-V3 approach) and [N] "Load balancing" item 3: selection on
// softmax score + bias, gates from the raw scores renormalised.  [G] "Load
// balancing and expert capacity": Switch routes each token to one expert.
#include "moe_internal.h"

#include <math.h>

namespace moe {

// --------------------------------------------------------------------------- router GEMM
//
// One wavefront computes a 16-token x (16*NB)-expert block with
// v_mfma_f32_16x16x32_bf16 over a slice of the d axis; `waves_k` wavefronts of
// the workgroup split d and their partial sums are added in a fixed order in
// LDS, so the result does not depend on timing.  The router weight is small
// (E x d) and stays in L2; x streams from HBM once.
//
// MFMA 16x16x32 operand layout (lane l): A row l%16, k = 8*(l/16)..+7;
// B column l%16, same k; D column l%16, rows 4*(l/16)..+3.
template <int NB>
__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ logit_bias, float* __restrict__ logits,
    int N, int d, int E, int waves_k) {
  extern __shared__ float red[];   // [(waves_k-1) * waves_m][16][16*NB]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int waves_m = 4 / waves_k;
  const int wm = wave / waves_k, wk = wave % waves_k;
  const int t0 = (blockIdx.x * waves_m + wm) * 16;
  const int r16 = lane & 15, kq = lane >> 4;

  int t = t0 + r16;
  if (t > N - 1) t = N - 1;
  const uint16_t* xa = x + (size_t)t * d + kq * 8;
  const uint16_t* wb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int e = nb * 16 + r16;
    if (e > E - 1) e = E - 1;           // columns past E are computed but never stored
    wb[nb] = w + (size_t)e * d + kq * 8;
  }
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = d / 32;
  const int per = (ksteps + waves_k - 1) / waves_k;
  const int ks0 = wk * per;
  const int ks1 = min(ksteps, ks0 + per);
  for (int ks = ks0; ks < ks1; ++ks) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(xa + ks * 32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(wb[nb] + ks * 32);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }

  const int cols = 16 * NB;
  if (waves_k > 1) {
    if (wk > 0) {
      float* dst = red + ((size_t)(wm * (waves_k - 1) + (wk - 1)) * 16) * cols;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(kq * 4 + i) * cols + nb * 16 + r16] = acc[nb][i];
    }
    __syncthreads();
    if (wk > 0) return;
    for (int j = 1; j < waves_k; ++j) {
      const float* src = red + ((size_t)(wm * (waves_k - 1) + (j - 1)) * 16) * cols;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] += src[(kq * 4 + i) * cols + nb * 16 + r16];
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + r16;
    if (e >= E) continue;
    const float lb = logit_bias ? logit_bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = t0 + kq * 4 + i;
      if (tt < N) logits[(size_t)tt * E + e] = acc[nb][i] + lb;
    }
  }
}

// fp32 storage: one thread per (token, expert), sequential fp32 FMA over d.
__global__ __launch_bounds__(256) void router_gemm_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ logit_bias,
    float* __restrict__ logits, int N, int d, int E) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)N * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * d;
  const float* wr = w + (size_t)e * d;
  float acc = 0.f;
  for (int j = 0; j < d; ++j) acc = fmaf(xr[j], wr[j], acc);
  logits[i] = acc + (logit_bias ? logit_bias[e] : 0.f);
}

template <int NB>
static hipError_t launch_router_bf16_nb(const moe_config& c, const void* x, const void* w,
                                        const float* lb, float* logits, hipStream_t s) {
  const int waves_k = NB <= 4 ? 4 : 2;
  const int waves_m = 4 / waves_k;
  const int N = (int)c.n_tokens;
  const int grid = (N + 16 * waves_m - 1) / (16 * waves_m);
  const size_t lds = (size_t)(waves_k - 1) * waves_m * 16 * 16 * NB * sizeof(float);
  hipLaunchKernelGGL(router_gemm_bf16_kernel<NB>, dim3(grid), dim3(256), lds, s,
                     (const uint16_t*)x, (const uint16_t*)w, lb, logits, N, c.d_model, c.n_experts,
                     waves_k);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const moe_config& c, const void* x, const void* w,
                              const float* logit_bias, float* logits, hipStream_t s) {
  if (c.n_tokens == 0) return hipSuccess;
  if (c.dtype == MOE_F32) {
    const size_t n = (size_t)c.n_tokens * c.n_experts;
    hipLaunchKernelGGL(router_gemm_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)x, (const float*)w, logit_bias, logits, (int)c.n_tokens,
                       c.d_model, c.n_experts);
    return hipGetLastError();
  }
  const int nb = (c.n_experts + 15) / 16;
  if (nb <= 1) return launch_router_bf16_nb<1>(c, x, w, logit_bias, logits, s);
  if (nb <= 2) return launch_router_bf16_nb<2>(c, x, w, logit_bias, logits, s);
  if (nb <= 4) return launch_router_bf16_nb<4>(c, x, w, logit_bias, logits, s);
  if (nb <= 8) return launch_router_bf16_nb<8>(c, x, w, logit_bias, logits, s);
  return launch_router_bf16_nb<16>(c, x, w, logit_bias, logits, s);
}

// --------------------------------------------------------------------------- top-k and gates
//
// A group of L lanes handles one token; lane gl of the group owns the V
// consecutive experts gl*V .. gl*V+V-1, so a lower lane always holds lower
// expert indices.  Each of the k rounds takes the group maximum of the
// per-lane best key (xor shuffles), ballots the lanes holding it and lets the
// lowest such lane win: exact ties go to the lower expert index.  Keys are
// fp64, formed from the fp32 logits and bias.  KM >= k bounds the unrolled
// selection rounds and the per-token arrays (kMaxTopK for every k kept the
// E = 256 kernel at 189 VGPRs, two wavefronts per SIMD).
template <int L, int V, int KM>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ zin, float* __restrict__ zout, const float* __restrict__ sel_bias,
    int N, int E, int k, int rule, int iters, int32_t* __restrict__ idx_out,
    float* __restrict__ gates_out, double* __restrict__ probsum_part) {
  constexpr int G = 64 / L;
  __shared__ double psum_lds[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / L, gl = lane % L, gbase = g * L;
  const uint64_t gmask = (L == 64) ? ~0ull : (((1ull << L) - 1ull) << gbase);
  const bool want_p = (rule != MOE_GATE_TOPK_SOFTMAX) || (probsum_part != nullptr);

  int ex[V];
  bool valid[V];
  double b[V], pacc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ex[v] = gl * V + v;
    valid[v] = ex[v] < E;
    b[v] = (sel_bias != nullptr && valid[v] && rule != MOE_GATE_SWITCH_TOP1) ? (double)sel_bias[ex[v]] : 0.0;
    pacc[v] = 0.0;
  }

  const int tokens_per_block = 4 * G * iters;
  for (int it = 0; it < iters; ++it) {
    const int t = blockIdx.x * tokens_per_block + (it * 4 + wave) * G + g;
    const bool tv = t < N;
    float z[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      z[v] = valid[v] ? (tv ? zin[(size_t)t * E + ex[v]] : 0.f) : -INFINITY;
      if (zout != nullptr && tv && valid[v]) zout[(size_t)t * E + ex[v]] = z[v];
    }
    double p[V];
    if (want_p) {
      float m = z[0];
#pragma unroll
      for (int v = 1; v < V; ++v) m = fmaxf(m, z[v]);
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, L));
      double sum = 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        p[v] = valid[v] ? exp((double)z[v] - (double)m) : 0.0;
        sum += p[v];
      }
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, L);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        p[v] = p[v] / sum;
        if (tv) pacc[v] += p[v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) p[v] = 0.0;
    }
    double key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const double kv = rule == MOE_GATE_SOFTMAX_RENORM ? p[v] + b[v] : (double)z[v] + b[v];
      key[v] = valid[v] ? kv : -INFINITY;
    }

    bool taken[V];
#pragma unroll
    for (int v = 0; v < V; ++v) taken[v] = false;
    int sel[KM];
    float zsel[KM];
    double psel[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      sel[j] = 0; zsel[j] = 0.f; psel[j] = 0.0;
      if (j < k) {
        double bk = -INFINITY;
        int bi = 0x7fffffff;
        float bz = 0.f;
        double bp = 0.0;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if (valid[v] && !taken[v] && (bi == 0x7fffffff || key[v] > bk)) {
            bk = key[v]; bi = ex[v]; bz = z[v]; bp = p[v];
          }
        }
        double gm = bk;
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) gm = fmax(gm, __shfl_xor(gm, off, L));
        const bool cand = (bi != 0x7fffffff) && (bk == gm);
        uint64_t mine = __ballot(cand) & gmask;
        if (mine == 0) mine = __ballot(bi != 0x7fffffff) & gmask;   // only with NaN keys
        const int wl = mine ? __builtin_ctzll(mine) : gbase;
        const int ew = __shfl(bi, wl);
        const float zw = __shfl(bz, wl);
        const double pw = __shfl(bp, wl);
        if (lane == wl) {
#pragma unroll
          for (int v = 0; v < V; ++v)
            if (ex[v] == ew) taken[v] = true;
        }
        sel[j] = ew; zsel[j] = zw; psel[j] = pw;
      }
    }

    if (tv) {
      double gate[KM];
      if (rule == MOE_GATE_TOPK_SOFTMAX) {
        double m = zsel[0];
#pragma unroll
        for (int j = 1; j < KM; ++j)
          if (j < k) m = fmax(m, (double)zsel[j]);
        double den = 0.0;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          gate[j] = j < k ? exp((double)zsel[j] - m) : 0.0;
          den += gate[j];
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) gate[j] /= den;
      } else if (rule == MOE_GATE_SOFTMAX_RENORM) {
        double den = 0.0;
#pragma unroll
        for (int j = 0; j < KM; ++j) den += j < k ? psel[j] : 0.0;
#pragma unroll
        for (int j = 0; j < KM; ++j) gate[j] = psel[j] / den;
      } else {
#pragma unroll
        for (int j = 0; j < KM; ++j) gate[j] = psel[j];
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k && (j % L) == gl) {   // k may exceed L
          idx_out[(size_t)t * k + j] = sel[j];
          gates_out[(size_t)t * k + j] = (float)gate[j];
        }
      }
    }
  }

  if (probsum_part == nullptr) return;
  // Per-expert sums: groups of this wave in order, then the four waves in order.
#pragma unroll
  for (int v = 0; v < V; ++v) {
    double tot = pacc[v];
    for (int gg = 1; gg < G; ++gg) tot += __shfl(pacc[v], gg * L + gl);
    if (g == 0 && valid[v]) psum_lds[wave][ex[v]] = tot;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const double s = ((psum_lds[0][e] + psum_lds[1][e]) + psum_lds[2][e]) + psum_lds[3][e];
    probsum_part[(size_t)blockIdx.x * E + e] = s;
  }
}

// Sum the per-block partials of expert e = blockIdx.x: lane l adds blocks
// l, l + 64, ... in order, then a fixed xor tree combines the lanes, so the
// result does not depend on timing.
__global__ __launch_bounds__(64) void probsum_reduce_kernel(const double* __restrict__ part, int nblk,
                                                            int E, float* __restrict__ probsum) {
  const int e = blockIdx.x, lane = threadIdx.x;
  double s = 0.0;
  for (int b = lane; b < nblk; b += 64) s += part[(size_t)b * E + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) probsum[e] = (float)s;
}

template <int L, int V, int KM>
static void launch_topk_lvk(const moe_config& c, const Workspace& W, const float* zin, float* zout,
                            const float* sel_bias, int32_t* idx, float* gates, double* part,
                            hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<L, V, KM>), dim3(W.topk_blocks), dim3(256), 0, s, zin, zout, sel_bias,
                     (int)c.n_tokens, c.n_experts, c.top_k, c.gate_rule, W.topk_iters, idx, gates, part);
}

template <int L, int V>
static void launch_topk_lv(const moe_config& c, const Workspace& W, const float* zin, float* zout,
                           const float* sel_bias, int32_t* idx, float* gates, double* part,
                           hipStream_t s) {
  const int k = c.top_k;
  if (k <= 2) launch_topk_lvk<L, V, 2>(c, W, zin, zout, sel_bias, idx, gates, part, s);
  else if (k <= 4) launch_topk_lvk<L, V, 4>(c, W, zin, zout, sel_bias, idx, gates, part, s);
  else if (k <= 8) launch_topk_lvk<L, V, 8>(c, W, zin, zout, sel_bias, idx, gates, part, s);
  else launch_topk_lvk<L, V, kMaxTopK>(c, W, zin, zout, sel_bias, idx, gates, part, s);
}

hipError_t launch_topk(const moe_config& c, const Workspace& W, const float* zin, float* zout,
                       const float* sel_bias, int32_t* idx, float* gates, float* probsum_part_f,
                       float* probsum, hipStream_t s) {
  double* part = probsum ? reinterpret_cast<double*>(probsum_part_f) : nullptr;
  if (c.n_tokens > 0) {
    const int E = c.n_experts;
    // L = topk_lanes(E) lanes per token, V = experts per lane
    if (E <= 8) launch_topk_lv<8, 1>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    else if (E <= 16) launch_topk_lv<8, 2>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    else if (E <= 32) launch_topk_lv<8, 4>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    else if (E <= 64) launch_topk_lv<8, 8>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    else if (E <= 128) launch_topk_lv<16, 8>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    else launch_topk_lv<64, 4>(c, W, zin, zout, sel_bias, idx, gates, part, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (probsum) {
    const int nblk = c.n_tokens > 0 ? W.topk_blocks : 0;
    hipLaunchKernelGGL(probsum_reduce_kernel, dim3(c.n_experts), dim3(64), 0, s, part, nblk, c.n_experts,
                       probsum);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
