// Gate-weighted combine into token order, the auxiliary load-balance loss and
// the aux-loss-free bias step.
//
// [L] "Concept / FFN swap": h + sum over the chosen experts of gate * expert(h);
// [G] "How an MoE layer works": the chosen experts' outputs are weighted by the
// normalised router scores and summed; [G] "Load balancing and expert
// capacity": tokens over capacity skip the layer's experts and continue along
// the residual connection.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr size_t kLastLevelCacheBytes = 256ull << 20;   // MI355X Infinity Cache (MALL)

template <typename T>
union Vec16 {
  uint4 u;
  T e[16 / sizeof(T)];
};

// One wavefront per token.  out = (residual + shared) + sum_j g_j * y[slot_pos_j],
// j ascending, fp32 accumulation, one rounding to the storage type at the end.
// STREAM: the expert rows are loaded and the output stored with nontemporal
// hints, for calls whose expert rows exceed the 256 MB last-level cache
// (DeepSeek-V3 shapes: 0.94 GB, 277 -> 229 us).  Below that size the rows
// the down projection just wrote still hit in that cache, and the hints cost
// (Mixtral prefill: 21 -> 25 us); a hint on only the loads or only the stores
// gains 2-3%.
// `parts` wavefronts share a token's row (each its own contiguous 1 / parts of
// the columns; same per-element arithmetic), so that a small batch (decode)
// still keeps every column's loads in flight at once.
// KM >= k bounds the unrolled slot loop.  All KM expert rows of a chunk are loaded before the
// first is used (a dropped slot, or one past k, loads row 0 and is not added), so a lane has
// KM + 2 loads in flight per chunk instead of waiting on each row in turn.
template <typename T, bool STREAM, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ gates, const T* __restrict__ res,
                                                      const T* __restrict__ sh, T* __restrict__ out, int N,
                                                      int d, int k, int parts) {
  constexpr int VEC = 16 / sizeof(T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  const int t = gw / parts, part = gw % parts;
  if (t >= N) return;
  const int span = d / parts, c_beg = part * span, c_end = c_beg + span;
  int pos[KM];
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
    g[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
  }
  const size_t trow = (size_t)t * d;
  if (d % VEC == 0) {
#pragma unroll 2
    for (int c = c_beg + lane * VEC; c < c_end; c += 64 * VEC) {   // two chunks in flight per lane
      Vec16<T> yb[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {   // no branch around the loads: slots past k and dropped slots read row 0
        const size_t yr = (size_t)(pos[j] >= 0 ? pos[j] : 0) * d + c;
        if (STREAM) {
          const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + yr));
          yb[j].u = uint4{raw.x, raw.y, raw.z, raw.w};
        } else {
          yb[j].u = *reinterpret_cast<const uint4*>(y + yr);
        }
      }
      float acc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
      if (res) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = Store<T>::load(res, trow + c + v);
      }
      if (sh) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += Store<T>::load(sh, trow + c + v);
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j >= k || pos[j] < 0) continue;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fmaf(g[j], Store<T>::load(yb[j].e, v), acc[v]);
      }
      Vec16<T> ob;
#pragma unroll
      for (int v = 0; v < VEC; ++v) Store<T>::store(ob.e, v, acc[v]);
      if (STREAM)
        __builtin_nontemporal_store(u32x4{ob.u.x, ob.u.y, ob.u.z, ob.u.w}, reinterpret_cast<u32x4*>(out + trow + c));
      else
        *reinterpret_cast<uint4*>(out + trow + c) = ob.u;
    }
  } else {
    for (int c = c_beg + lane; c < c_end; c += 64) {
      float acc = res ? Store<T>::load(res, trow + c) : 0.f;
      if (sh) acc += Store<T>::load(sh, trow + c);
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (pos[j] >= 0) acc = fmaf(g[j], Store<T>::load(y, (size_t)pos[j] * d + c), acc);
      Store<T>::store(out, trow + c, acc);
    }
  }
}

// Top-1 routing with the combine fused into the down projection: a token whose
// slot was dropped gets out = [residual] + [shared_y] (the same fp32 sum and
// single rounding as combine_kernel).  One wavefront per token, 16-byte lanes.
__global__ __launch_bounds__(256) void combine_dropped_kernel(const int32_t* __restrict__ slot_pos,
                                                              const uint16_t* __restrict__ res,
                                                              const uint16_t* __restrict__ sh,
                                                              uint16_t* __restrict__ out, int N, int d) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N || slot_pos[t] >= 0) return;
  const size_t trow = (size_t)t * d;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.f;
    if (res) {
      Vec8 r;
      r.u = *reinterpret_cast<const uint4*>(res + trow + c);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] = bf16_to_f32(r.e[v]);
    }
    if (sh) {
      Vec8 y;
      y.u = *reinterpret_cast<const uint4*>(sh + trow + c);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] += bf16_to_f32(y.e[v]);
    }
    *reinterpret_cast<uint4*>(out + trow + c) = pack_bf16x8(acc);
  }
}

hipError_t launch_combine_dropped(const moe_config& c, const int32_t* slot_pos, const void* residual,
                                  const void* shared_y, void* out, hipStream_t s) {
  const int N = (int)c.n_tokens;
  if (N == 0) return hipSuccess;
  if (c.top_k != 1 || c.d_model % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_dropped_kernel, dim3((N + 3) / 4), dim3(256), 0, s, slot_pos,
                     (const uint16_t*)residual, (const uint16_t*)shared_y, (uint16_t*)out, N, c.d_model);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* slot_pos,
                          const float* gates, const void* residual, const void* shared_y,
                          void* out, hipStream_t s) {
  const int N = (int)c.n_tokens;
  if (N == 0) return hipSuccess;
  const size_t esz = c.dtype == MOE_BF16 ? 2 : 4;
  // wavefronts per token: up to 8, while the batch has fewer than 1024 tokens, each keeping whole
  // 16-byte chunks of 64 lanes (a column count that does not split that way keeps one wavefront)
  const int chunk = 64 * (int)(16 / esz);
  int parts = 1;
  while (parts < 8 && (long long)N * parts < 1024 && c.d_model % (2 * parts * chunk) == 0) parts *= 2;
  const dim3 grid((unsigned)(((long long)N * parts + 3) / 4));
  const bool stream = (size_t)N * c.top_k * c.d_model * esz > kLastLevelCacheBytes;
  auto go = [&](auto kern, auto* tp) {
    using T = std::remove_pointer_t<decltype(tp)>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const T*)y_perm, slot_pos, gates, (const T*)residual,
                       (const T*)shared_y, (T*)out, N, c.d_model, c.top_k, parts);
  };
  auto by_k = [&](auto t_s, auto s_s) {
    using T = decltype(t_s);
    constexpr bool S = decltype(s_s)::value;
    const int k = c.top_k;
    if (k <= 2) go(combine_kernel<T, S, 2>, (T*)nullptr);
    else if (k <= 4) go(combine_kernel<T, S, 4>, (T*)nullptr);
    else if (k <= 8) go(combine_kernel<T, S, 8>, (T*)nullptr);
    else go(combine_kernel<T, S, kMaxTopK>, (T*)nullptr);
  };
  if (c.dtype == MOE_BF16) {
    if (stream) by_k(uint16_t{}, std::true_type{});
    else by_k(uint16_t{}, std::false_type{});
  } else {
    if (stream) by_k(float{}, std::true_type{});
    else by_k(float{}, std::false_type{});
  }
  return hipGetLastError();
}

// [L] "The load balance problem", DeepSeek-V3 approach: after a step, an
// expert above its target load moves its bias down by gamma, one below moves
// it up.  load - target is compared as counts * E against N * k in integers.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                          long long nk, float gamma,
                                                          const float* sel_bias_in, float* sel_bias_out,
                                                          int8_t* __restrict__ signs) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const long long diff = (long long)counts[e] * E - nk;
    const int sgn = (diff > 0) - (diff < 0);
    if (signs) signs[e] = (int8_t)sgn;
    if (sel_bias_out) sel_bias_out[e] = sel_bias_in[e] - gamma * (float)sgn;
  }
}

hipError_t launch_bias_update(const moe_config& c, const int32_t* counts, float gamma,
                              const float* sel_bias_in, float* sel_bias_out, int8_t* signs,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, counts, c.n_experts,
                     (long long)c.n_tokens * c.top_k, gamma, sel_bias_in, sel_bias_out, signs);
  return hipGetLastError();
}

// [G] "Load balancing and expert capacity" (Switch's extra loss term, smallest
// when tokens and probabilities spread evenly): aux = E * sum_e f_e * P_e with
// f_e = counts_e / (N k), P_e = probsum_e / N.  Fixed-order reduction.
__global__ __launch_bounds__(256) void aux_loss_kernel(const int32_t* __restrict__ counts,
                                                       const float* __restrict__ probsum, int E,
                                                       long long N, int k, float* __restrict__ aux) {
  __shared__ double wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double term = 0.0;
  if (N > 0 && tid < E)
    term = ((double)counts[tid] / (double)(N * k)) * ((double)probsum[tid] / (double)N);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) term += __shfl_xor(term, off);
  if (lane == 0) wsum[wave] = term;
  __syncthreads();
  if (tid == 0) *aux = (float)((double)E * (((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]));
}

hipError_t launch_aux_loss(const moe_config& c, const int32_t* counts, const float* probsum,
                           float* aux, hipStream_t s) {
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, s, counts, probsum, c.n_experts,
                     (long long)c.n_tokens, c.top_k, aux);
  return hipGetLastError();
}

}  // namespace moe
