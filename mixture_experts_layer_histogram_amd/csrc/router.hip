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

#include <type_traits>

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
// A group of L lanes (8, 16 or 64, aligned) handles one token; lane gl of the
// group owns the V consecutive experts gl*V .. gl*V+V-1, so a lower lane always
// holds lower expert indices.  Each of the k rounds takes the group maximum of
// the per-lane best key; among the lanes holding it the lowest expert index
// wins (a group minimum), so exact ties go to the lower expert index, and the
// winner's logit and probability reach the group by an OR of the one lane's
// bits.  Keys are fp64, formed from the fp32 logits and bias.  KM >= k bounds
// the unrolled selection rounds and the per-token arrays (kMaxTopK for every k
// kept the E = 256 kernel at 189 VGPRs, two wavefronts per SIMD).
//
// The group reductions move data between lanes with DPP within each row of 16
// lanes (quad permutations, then the half-row and row mirrors: after each step
// a lane and its partner hold the same pair, so every lane ends with the same
// bits) and, for 64-lane groups, read the four row results with v_readlane.
// (Through ds_bpermute, each of the 6 steps of a 64-lane reduction waited on an
// LDS round trip.)
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = dpp_i32<CTRL>((int)(unsigned)(b & 0xffffffffll)), hi = dpp_i32<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(unsigned)(b & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

// op over the L-lane group; T is int, float or double
template <int L, class T, class Op>
__device__ __forceinline__ T group_reduce(T x, Op op) {
  static_assert(L == 8 || L == 16 || L == 64, "group of 8, 16 or 64 lanes");
  auto mv = [](T v, auto ctrl) -> T {
    constexpr int C = decltype(ctrl)::value;
    if constexpr (sizeof(T) == 8) return dpp_f64<C>(v);
    else if constexpr (std::is_same<T, float>::value) return __int_as_float(dpp_i32<C>(__float_as_int(v)));
    else return dpp_i32<C>(v);
  };
  x = op(x, mv(x, std::integral_constant<int, kDppQuadXor1>{}));
  x = op(x, mv(x, std::integral_constant<int, kDppQuadXor2>{}));
  x = op(x, mv(x, std::integral_constant<int, kDppRowHalfMirror>{}));
  if (L >= 16) x = op(x, mv(x, std::integral_constant<int, kDppRowMirror>{}));
  if (L == 64) {
    T r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(T) == 8) r[i] = readlane_f64(x, 16 * i);
      else if constexpr (std::is_same<T, float>::value)
        r[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16 * i));
      else r[i] = __builtin_amdgcn_readlane(x, 16 * i);
    }
    x = op(op(r[0], r[1]), op(r[2], r[3]));
  }
  return x;
}

template <int L, int V, int KM>
__device__ __forceinline__ void select_token(const float (&z)[V], const int (&ex)[V], const bool (&valid)[V],
                                             const double (&b)[V], int k, int rule, bool want_p, bool tv, int t,
                                             int lane, int gl, int gbase, uint64_t gmask,
                                             int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
                                             double (&p)[V]) {
  if (want_p) {
    float m = z[0];
#pragma unroll
    for (int v = 1; v < V; ++v) m = fmaxf(m, z[v]);
    m = group_reduce<L>(m, [](float a, float c) { return fmaxf(a, c); });
    double sum = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      p[v] = valid[v] ? exp((double)z[v] - (double)m) : 0.0;
      sum += p[v];
    }
    sum = group_reduce<L>(sum, [](double a, double c) { return a + c; });
#pragma unroll
    for (int v = 0; v < V; ++v) p[v] = p[v] / sum;
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
      const double gm = group_reduce<L>(bk, [](double a, double c) { return fmax(a, c); });
      const bool cand = (bi != 0x7fffffff) && (bk == gm);
      auto imin = [](int a, int c) { return a < c ? a : c; };
      int ew = group_reduce<L>(cand ? bi : 0x7fffffff, imin);
      if (ew == 0x7fffffff) ew = group_reduce<L>(bi, imin);   // only with NaN keys: the lowest open expert
      const bool win = bi == ew && bi != 0x7fffffff;          // one lane of the group
      auto ior = [](int a, int c) { return a | c; };
      const long long pb = __double_as_longlong(bp);
      const float zw = __int_as_float(group_reduce<L>(win ? __float_as_int(bz) : 0, ior));
      const int plo = group_reduce<L>(win ? (int)(unsigned)(pb & 0xffffffffll) : 0, ior);
      const int phi = group_reduce<L>(win ? (int)(pb >> 32) : 0, ior);
      const double pw = __longlong_as_double(((long long)phi << 32) | (unsigned)plo);
      if (win) {
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

// Per-expert probability sums of one workgroup: in each wave the groups in
// order, then the waves in order (`nw` waves hold tokens).
template <int L, int V>
__device__ __forceinline__ void probsum_block(const double (&pacc)[V], const int (&ex)[V], const bool (&valid)[V],
                                              int wave, int nw, int lane, int gl, int E,
                                              double (*psum_lds)[kMaxExperts], double* __restrict__ out) {
  constexpr int G = 64 / L;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    double tot = pacc[v];
    for (int gg = 1; gg < G; ++gg) tot += __shfl(pacc[v], gg * L + gl);
    if (wave < nw && lane < L && valid[v]) psum_lds[wave][ex[v]] = tot;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double s = psum_lds[0][e];
    for (int w = 1; w < nw; ++w) s += psum_lds[w][e];
    out[(size_t)blockIdx.x * E + e] = s;
  }
}

// Logit of token t, experts 4 gl .. 4 gl + 3, from the logits GEMM's K-part
// partials: the tile's parts summed in part order, then the bias (the order of
// the GEMM's fix-up, so the values are the ones it would have written); rows of
// unsplit tiles are final already.  Writes the completed logits.
__device__ __forceinline__ float4 logits_from_parts(const LogitParts zp, int t, int gl, int E) {
  const int col = 4 * gl;
  const float* base = nullptr;
  int parts = 0, stride = 0;
  if (t < zp.nb * 256) {
    const int i = t >> 8;
    if (i >= zp.full_b) {
      base = zp.part_big + ((size_t)(i - zp.full_b) * zp.s_b * zp.rows_big + (t & 255)) * zp.ld;
      parts = zp.s_b;
      stride = zp.rows_big * zp.ld;
    }
  } else {
    const int j = (t - zp.nb * 256) >> 6;
    if (j >= zp.full_s) {
      base = zp.part_small + ((size_t)(j - zp.full_s) * zp.s_s * 64 + ((t - zp.nb * 256) & 63)) * zp.ld;
      parts = zp.s_s;
      stride = 64 * zp.ld;
    }
  }
  float4 z;
  if (base == nullptr) return *reinterpret_cast<const float4*>(zp.logits + (size_t)t * E + col);
  z = *reinterpret_cast<const float4*>(base + col);
  for (int q = 1; q < parts; ++q) {
    const float4 x = *reinterpret_cast<const float4*>(base + (size_t)q * stride + col);
    z.x += x.x; z.y += x.y; z.z += x.z; z.w += x.w;
  }
  if (zp.bias) {
    const float4 b = *reinterpret_cast<const float4*>(zp.bias + col);
    z.x += b.x; z.y += b.y; z.z += b.z; z.w += b.w;
  }
  *reinterpret_cast<float4*>(zp.logits + (size_t)t * E + col) = z;
  return z;
}

template <int L, int V, int KM, bool PARTS = false>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ zin, float* __restrict__ zout, const float* __restrict__ sel_bias,
    int N, int E, int k, int rule, int iters, int32_t* __restrict__ idx_out,
    float* __restrict__ gates_out, double* __restrict__ probsum_part, LogitParts zp = {}) {
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
    if (PARTS) {   // L = 64, V = 4, E a multiple of 4: the lane's experts are one float4
      static_assert(!PARTS || V == 4, "one float4 of logits per lane");
      float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tv && valid[0]) q = logits_from_parts(zp, t, gl, E);
      z[0] = valid[0] ? q.x : -INFINITY;
      z[1 % V] = valid[1 % V] ? q.y : -INFINITY;
      z[2 % V] = valid[2 % V] ? q.z : -INFINITY;
      z[3 % V] = valid[3 % V] ? q.w : -INFINITY;
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        z[v] = valid[v] ? (tv ? zin[(size_t)t * E + ex[v]] : 0.f) : -INFINITY;
        if (zout != nullptr && tv && valid[v]) zout[(size_t)t * E + ex[v]] = z[v];
      }
    }
    double p[V];
    select_token<L, V, KM>(z, ex, valid, b, k, rule, want_p, tv, t, lane, gl, gbase, gmask, idx_out, gates_out, p);
    if (tv) {
#pragma unroll
      for (int v = 0; v < V; ++v) pacc[v] += p[v];
    }
  }

  if (probsum_part == nullptr) return;
  // Per-expert sums: groups of this wave in order, then the four waves in order.
  probsum_block<L, V>(pacc, ex, valid, wave, 4, lane, gl, E, psum_lds, probsum_part);
}

// --------------------------------------------------------------------------- fused router
//
// Router GEMM, softmax, top-k and gates in one kernel for E <= 64 ([L] Step 1:
// one linear layer, then top-k and softmax; [G] "How an MoE layer works").  A
// workgroup of 8 wavefronts takes TM = 16 MB tokens at a time (16 for E <= 16,
// else 64, which halves the router weight's L2 traffic per token): each wavefront
// multiplies the tokens' rows by all E router rows (MFMA 16x16x32, NB blocks
// of 16 experts) over its eighth of d; the eight partial tiles are added in
// LDS in wavefront order (+ logit bias), so the logits do not depend on
// timing; then 8-lane groups select from the logits in LDS exactly as
// topk_kernel does (fp64 keys, ties to the lower index), and the workgroup
// keeps its per-expert probability sums for probsum_reduce_kernel.  x streams
// from HBM once; the router weight (E d bf16) is read from L2 once per TM
// tokens.  The logits are still written (the parity hook compares them).
constexpr int kRouteWaves = 8;

template <int NB, int MB, int KM>
__global__ __launch_bounds__(512) void route_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ logit_bias,
    const float* __restrict__ sel_bias, float* __restrict__ logits, int N, int d, int E, int k, int rule,
    int32_t* __restrict__ idx_out, float* __restrict__ gates_out, double* __restrict__ probsum_part) {
  constexpr int TM = 16 * MB, EP = 16 * NB, L = 8, V = EP / L;
  __shared__ float red[kRouteWaves][TM][EP];
  __shared__ double psum_lds[kRouteWaves][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int g = lane / L, gl = lane % L, gbase = g * L;
  const uint64_t gmask = ((1ull << L) - 1ull) << gbase;
  const bool want_p = (rule != MOE_GATE_TOPK_SOFTMAX) || (probsum_part != nullptr);
  const int ksteps = d / 32;
  const int per = (ksteps + kRouteWaves - 1) / kRouteWaves;
  const int ks0 = wave * per, ks1 = min(ksteps, ks0 + per);

  const uint16_t* wb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wb[nb] = w + (size_t)min(nb * 16 + r16, E - 1) * d + kq * 8;
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

  const int groups = (N + TM - 1) / TM;
  for (int grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int t0 = grp * TM;
    // 1. this wavefront's share of d for all TM tokens and all experts
    const uint16_t* xa[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xa[mb] = x + (size_t)min(t0 + mb * 16 + r16, N - 1) * d + kq * 8;
    f32x4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // UNR K steps of loads in flight (as many as the registers allow), then the remainder one by one
    constexpr int UNR = MB + NB <= 2 ? 16 : (MB + NB <= 4 ? 8 : 4);
    auto kstep = [&](const bf16x8 (&a)[MB], const bf16x8 (&bb)[NB]) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], bb[nb], acc[mb][nb], 0, 0, 0);
    };
    int ks = ks0;
    for (; ks + UNR <= ks1; ks += UNR) {
      bf16x8 a[UNR][MB], bb[UNR][NB];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[u][mb] = *reinterpret_cast<const bf16x8*>(xa[mb] + (ks + u) * 32);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bb[u][nb] = *reinterpret_cast<const bf16x8*>(wb[nb] + (ks + u) * 32);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) kstep(a[u], bb[u]);
    }
    for (; ks < ks1; ++ks) {
      bf16x8 a[MB], bb[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const bf16x8*>(xa[mb] + ks * 32);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bb[nb] = *reinterpret_cast<const bf16x8*>(wb[nb] + ks * 32);
      kstep(a, bb);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][mb * 16 + kq * 4 + i][nb * 16 + r16] = acc[mb][nb][i];
    __syncthreads();
    // 2. partial tiles added in wavefront order, + logit bias; logits out
    for (int i = threadIdx.x; i < TM * EP; i += blockDim.x) {
      const int row = i / EP, col = i % EP;
      float z = red[0][row][col];
#pragma unroll
      for (int ww = 1; ww < kRouteWaves; ++ww) z += red[ww][row][col];
      if (col < E) {
        if (logit_bias) z += logit_bias[col];
        if (t0 + row < N) logits[(size_t)(t0 + row) * E + col] = z;
      }
      red[0][row][col] = z;
    }
    __syncthreads();
    // 3. selection: token t0 + 8 wave + g of the group
    const int tk = wave * (64 / L) + g;
    if (wave < TM / (64 / L)) {
      const int t = t0 + tk;
      const bool tv = t < N;
      float z[V];
#pragma unroll
      for (int v = 0; v < V; ++v) z[v] = valid[v] ? (tv ? red[0][tk][ex[v]] : 0.f) : -INFINITY;
      double p[V];
      select_token<L, V, KM>(z, ex, valid, b, k, rule, want_p, tv, t, lane, gl, gbase, gmask, idx_out, gates_out,
                             p);
      if (tv) {
#pragma unroll
        for (int v = 0; v < V; ++v) pacc[v] += p[v];
      }
    }
    __syncthreads();   // red is rewritten by the next group
  }
  if (probsum_part == nullptr) return;
  probsum_block<L, V>(pacc, ex, valid, wave, TM / (64 / L), lane, gl, E, psum_lds, probsum_part);
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

template <int NB, int MB>
static void launch_route_fused_nm(const moe_config& c, const Workspace& W, const void* x, const void* w,
                                  const float* lb, const float* sel_bias, float* logits, int32_t* idx, float* gates,
                                  double* part, hipStream_t s) {
  const int k = c.top_k;
  const dim3 grid(W.route_blocks), block(64 * kRouteWaves);
  const uint16_t *xx = (const uint16_t*)x, *ww = (const uint16_t*)w;
  const int N = (int)c.n_tokens;
  if (k <= 2)
    hipLaunchKernelGGL((route_fused_kernel<NB, MB, 2>), grid, block, 0, s, xx, ww, lb, sel_bias, logits, N,
                       c.d_model, c.n_experts, k, c.gate_rule, idx, gates, part);
  else if (k <= 4)
    hipLaunchKernelGGL((route_fused_kernel<NB, MB, 4>), grid, block, 0, s, xx, ww, lb, sel_bias, logits, N,
                       c.d_model, c.n_experts, k, c.gate_rule, idx, gates, part);
  else if (k <= 8)
    hipLaunchKernelGGL((route_fused_kernel<NB, MB, 8>), grid, block, 0, s, xx, ww, lb, sel_bias, logits, N,
                       c.d_model, c.n_experts, k, c.gate_rule, idx, gates, part);
  else
    hipLaunchKernelGGL((route_fused_kernel<NB, MB, kMaxTopK>), grid, block, 0, s, xx, ww, lb, sel_bias, logits, N,
                       c.d_model, c.n_experts, k, c.gate_rule, idx, gates, part);
}

bool route_fused_supported(const moe_config& c) { return c.dtype == MOE_BF16 && c.n_experts <= 64; }

hipError_t launch_route_fused(const moe_config& c, const Workspace& W, const void* x, const void* w,
                              const float* logit_bias, const float* sel_bias, float* logits, int32_t* idx,
                              float* gates, float* probsum_part_f, float* probsum, hipStream_t s) {
  if (!route_fused_supported(c)) return hipErrorInvalidValue;
  double* part = probsum ? reinterpret_cast<double*>(probsum_part_f) : nullptr;
  if (c.n_tokens > 0) {
    const int nb = (c.n_experts + 15) / 16;
    if (nb <= 1) launch_route_fused_nm<1, 1>(c, W, x, w, logit_bias, sel_bias, logits, idx, gates, part, s);
    else if (nb <= 2) launch_route_fused_nm<2, 4>(c, W, x, w, logit_bias, sel_bias, logits, idx, gates, part, s);
    else launch_route_fused_nm<4, 4>(c, W, x, w, logit_bias, sel_bias, logits, idx, gates, part, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (probsum) {
    const int nblk = c.n_tokens > 0 ? W.route_blocks : 0;
    hipLaunchKernelGGL(probsum_reduce_kernel, dim3(c.n_experts), dim3(64), 0, s, part, nblk, c.n_experts, probsum);
    return hipGetLastError();
  }
  return hipSuccess;
}

bool topk_from_parts_supported(const moe_config& c) {
  return c.n_experts > 128 && c.n_experts <= 256 && c.n_experts % 4 == 0;
}

hipError_t launch_topk_from_parts(const moe_config& c, const Workspace& W, const LogitParts& zp,
                                  const float* sel_bias, int32_t* idx, float* gates, float* probsum_part_f,
                                  float* probsum, hipStream_t s) {
  if (!topk_from_parts_supported(c) || topk_lanes(c.n_experts) != 64) return hipErrorInvalidValue;
  double* part = probsum ? reinterpret_cast<double*>(probsum_part_f) : nullptr;
  if (c.n_tokens > 0) {
    const int k = c.top_k;
    const dim3 grid(W.topk_blocks), block(256);
    const int N = (int)c.n_tokens, E = c.n_experts;
#define MOE_TOPK_PARTS(KMV)                                                                                  \
  hipLaunchKernelGGL((topk_kernel<64, 4, KMV, true>), grid, block, 0, s, nullptr, nullptr, sel_bias, N, E, k, \
                     c.gate_rule, W.topk_iters, idx, gates, part, zp)
    if (k <= 2) MOE_TOPK_PARTS(2);
    else if (k <= 4) MOE_TOPK_PARTS(4);
    else if (k <= 8) MOE_TOPK_PARTS(8);
    else MOE_TOPK_PARTS(kMaxTopK);
#undef MOE_TOPK_PARTS
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (probsum) {
    const int nblk = c.n_tokens > 0 ? W.topk_blocks : 0;
    hipLaunchKernelGGL(probsum_reduce_kernel, dim3(c.n_experts), dim3(64), 0, s, part, nblk, c.n_experts, probsum);
    return hipGetLastError();
  }
  return hipSuccess;
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
