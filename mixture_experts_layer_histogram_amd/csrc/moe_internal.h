// Internal declarations shared by the HIP translation units of libmoe_hip.
// Device helpers (bf16 conversion, wave reductions) and the host-side launch
// functions each kernel file exports to the C-ABI layer in moe_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kHistSlotsPerBlock = 1024;   // slots per workgroup in the histogram pass

// ----------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 in one word (lo in the low half), round to nearest even, NaN
// stays NaN: gfx950's packed conversion, one instruction for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return static_cast<uint16_t>(pack_bf16x2(f, f)); }

// Eight fp32 values -> eight bf16, one 16-byte vector.
__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// Eight bf16 values as one 16-byte load or store.
union Vec8 {
  uint4 u;
  uint16_t e[8];
};

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// u sigmoid(u), the sigmoid as the hardware reciprocal of 1 + 2^(-u log2 e) (each step within
// about an fp32 ulp, far below the bf16 rounding that follows; a divide costs 11 instructions)
__device__ __forceinline__ float silu_f(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * -1.44269504088896341f));
}
// GELU u Phi(u) = (u / 2) erfc(-u / sqrt 2), erfc from the Chebyshev fit of Numerical Recipes (section
// 6.2, "erfcc"): for z >= 0, erfc z = t exp(-z^2 + P(t)), t = 1 / (1 + z / 2), P of degree 9, with a
// fractional error below 1.2e-7 everywhere; erfc(-z) = 2 - erfc z.  The hardware reciprocal and exp2
// serve; evaluated in fp32 it changes one bf16 rounding in about 10^4 against the exact GELU, and
// costs a third of the library erfc's instructions.
__device__ __forceinline__ float gelu_f(float u) {
  const float z = u * -0.70710678118654752f, az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, az, 1.0f));
  float q = 0.17087277f;
  q = fmaf(q, t, -0.82215223f);
  q = fmaf(q, t, 1.48851587f);
  q = fmaf(q, t, -1.13520398f);
  q = fmaf(q, t, 0.27886807f);
  q = fmaf(q, t, -0.18628806f);
  q = fmaf(q, t, 0.09678418f);
  q = fmaf(q, t, 0.37409196f);
  q = fmaf(q, t, 1.00002368f);
  q = fmaf(q, t, -1.26551223f);
  const float r = t * __builtin_amdgcn_exp2f((q - az * az) * 1.44269504088896341f);
  return 0.5f * u * (z >= 0.f ? r : 2.0f - r);
}

// Top-k blocking: L lanes per token (each owning E / L consecutive experts, at
// most 8), so a wavefront routes 64 / L tokens at once.
inline int topk_lanes(int E) { return E <= 64 ? 8 : (E <= 128 ? 16 : 64); }

// Per-expert capacity C = floor(cf * N / E) in double (0x7fffffff when unlimited).
inline int capacity_of(const moe_config& c) {
  if (!(c.capacity_factor > 0.f)) return 0x7fffffff;
  const double cap = (double)c.capacity_factor * (double)c.n_tokens / (double)c.n_experts;
  return cap >= 2147483647.0 ? 0x7fffffff : (int)cap;
}

// Rows of the expert-ordered buffers (perm, x_perm, h, y): N k packed, E C padded.
inline long long expert_rows(const moe_config& c) {
  return c.capacity_layout == MOE_CAPACITY_PADDED ? (long long)c.n_experts * capacity_of(c)
                                                  : c.n_tokens * (long long)c.top_k;
}

// ----------------------------------------------------------------- workspace

struct Workspace {
  // scratch used by the step entry points (placed first)
  size_t probsum_part, hist_rank, hist_blocks, tiles, tiles_small, tiles_sh, tiles_sh_small, gemm_partials;
  // buffers moe_forward keeps when the caller passes no output pointer
  size_t logits, topk_idx, gates, probsum, counts, offsets, perm, slot_pos, drop_count,
         aux, signs, x_perm, h, y, h_sh, y_sh;
  size_t total;
  int topk_blocks, topk_tokens_per_block, topk_iters, hist_blocks_n, max_tiles, max_tiles_small, max_tiles_sh,
      max_tiles_sh_small, route_blocks;
};

// Layout of the workspace for one config (host).
Workspace workspace_layout(const moe_config& c);

// ----------------------------------------------------------------- launches (host)

hipError_t launch_router_gemm(const moe_config& c, const void* x, const void* w,
                              const float* logit_bias, float* logits, hipStream_t s);
// Router GEMM + softmax + top-k + gates in one kernel (bf16 storage, E <= 64).
bool route_fused_supported(const moe_config& c);
hipError_t launch_route_fused(const moe_config& c, const Workspace& W, const void* x, const void* w,
                              const float* logit_bias, const float* sel_bias, float* logits, int32_t* idx,
                              float* gates, float* probsum_part, float* probsum, hipStream_t s);
hipError_t launch_topk(const moe_config& c, const Workspace& L, const float* z_in, float* z_out,
                       const float* sel_bias, int32_t* idx, float* gates, float* probsum_part,
                       float* probsum, hipStream_t s);
// Logits left by the grouped GEMM in its fp32-logits mode without its fix-up (one dense
// segment of N rows, E <= 256 columns): rows of unsplit tiles are final in `logits`; the
// rows of split tiles are the sum, in part order, of their K-part partial tiles, + bias.
struct LogitParts {
  float* logits;                 // [N, E]: read for unsplit rows, written for split rows
  const float* part_big;         // [slot][256 rows][256 columns] fp32
  const float* part_small;       // [slot][64 rows][256 columns] fp32
  const float* bias;             // logit bias [E] or null
  int nb, full_b, s_b;           // 256-row tiles; the first full_b unsplit; s_b K-parts each after them
  int ns, full_s, s_s;           // 64-row tiles after row 256 nb, likewise
  int ld;                        // columns of a partial-tile row
  int rows_big;                  // rows of a 256-row tile's partial slot
};
// Selection (top-k, gates, probability sums) that first completes the logits from the
// K-part partials of the logits GEMM (E in (128, 256]: 64 lanes of 4 experts per token).
bool topk_from_parts_supported(const moe_config& c);
hipError_t launch_topk_from_parts(const moe_config& c, const Workspace& L, const LogitParts& z,
                                  const float* sel_bias, int32_t* idx, float* gates, float* probsum_part,
                                  float* probsum, hipStream_t s);

hipError_t launch_permute(const moe_config& c, const Workspace& L, const int32_t* topk_idx,
                          const void* x, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* slot_pos, int64_t* drop_count, void* x_perm,
                          int32_t* hist_rank, int32_t* hist_blocks, hipStream_t s);

// GEMM modes
enum GemmMode { MODE_SWIGLU_UP = 0, MODE_GELU_UP = 1, MODE_DOWN = 2, MODE_LOGITS = 3 };

// Grouped GEMM over ragged segments [offsets[e], offsets[e+1]) of `a`.
//   up   : h[r, :F]  = act(a[r, :K] W1_e^T [, a W3_e^T] [+ b1_e])
//   down : y[r, :Nn] = a[r, :K] W2_e^T [+ b2_e]
//   logits (one segment): z[r, :Nn] = a[r, :K] W^T [+ bias_f32] stored as fp32 (the router)
// `offsets` has n_seg+1 entries; `tiles` is scratch for the device-built tile list.
// With `perm` (up only), row r of the expert order is row perm[r] / gather_k
// of `a`, which then holds a_rows token rows.
struct GroupedGemmArgs {
  int mode;
  int dtype;
  int n_seg;
  int max_rows;          // upper bound on offsets[n_seg] (host-known)
  int K;                 // reduction length (d for up, F for down)
  int Nn;                // output columns (F for up, d for down)
  const void* a;
  const int32_t* perm;   // gather (up only): expert-order row -> slot id, or NULL
  int gather_k;          // gather: slots per token
  int a_rows;            // gather: rows of `a`
  const int32_t* offsets;
  const void* w;         // W1 (up) or W2 (down): [n_seg, Nn, K]
  const void* w3;        // SwiGLU up only
  const void* bias;      // b1 (up) / b2 (down) or NULL: [n_seg, Nn]
  void* out;             // [rows, Nn]
  void* pre;             // up modes, bf16: pre-activations [n_mat][max_rows, Nn] (x W1^T (+ b1) [, x W3^T]) or NULL
  // down mode, bf16, top-1 routing: gate-weighted combine in the epilogue instead of writing `out`:
  // out_tok[t] = [residual_t] + [shared_y_t] + gate_t * Y_row for the row whose slot is t = comb_perm[row]
  const int32_t* comb_perm;
  const float* comb_gates;
  const void* comb_residual;
  const void* comb_shared;
  void* comb_out;
  bool fp8;              // weights are E4M3 codes (w8, w8_3) with row scales (64-row tiles only)
  bool no_fixup;         // MODE_LOGITS: leave the K-part partials for launch_topk_from_parts
  const uint8_t* w8;     // fp8 W1 (up) or W2 (down): [n_seg, Nn, K]
  const uint8_t* w8_3;   // fp8 W3 (SwiGLU up)
  const float* scale1;   // row scales of w8 [n_seg, Nn]
  const float* scale3;   // row scales of w8_3
  float* out_f32;        // MODE_LOGITS output [rows, Nn]
  const float* bias_f32; // MODE_LOGITS bias [Nn] or NULL
  int32_t* tiles;        // scratch: 256-row tile list (4 header ints + 8 ints per tile)
  int max_tiles;
  int32_t* tiles_small;  // scratch: 64-row tile list
  int max_tiles_small;
  float* partials;       // scratch for K-split partial tiles (grouped_gemm_partials_bytes())
};
hipError_t launch_grouped_gemm(const GroupedGemmArgs& g, hipStream_t s);
// The K-part plan of a dense MODE_LOGITS call (what its no_fixup launch leaves in g.partials).
LogitParts logits_parts(const GroupedGemmArgs& g);
int grouped_gemm_max_tiles(int max_rows, int n_seg);
int grouped_gemm_max_small_tiles(int max_rows, int n_seg);
size_t grouped_gemm_partials_bytes();
size_t grouped_gemm_gather_max_bytes();   // largest token matrix (bytes) the bf16 gather path addresses

// Per-row fp8 (E4M3) quantisation of a bf16 [rows, cols] matrix: codes and fp32 scales.
hipError_t launch_quantize_fp8(const uint16_t* w, long long rows, int cols, uint8_t* q, float* scales,
                               hipStream_t s);

// Backward kernels (backward.hip); bf16 storage.
hipError_t launch_combine_backward(const moe_config& c, const void* dout, const void* y, const int32_t* slot_pos,
                                   const float* gates, float* dg, void* dy, hipStream_t s);
hipError_t launch_act_backward(bool swiglu, const void* a1, const void* a3, const void* dh, long long rows, int F,
                               void* h, void* da, hipStream_t s);
hipError_t launch_segment_colsum(const void* a, int lda, int col0, int ncols, const int32_t* offsets,
                                 const int32_t* perm, int dense_rows, int n_seg, float* out, hipStream_t s);
size_t colsum_part_floats(int rows, int cols);   // scratch of launch_colsum_f32
hipError_t launch_colsum_f32(const float* a, int rows, int cols, float* part, float* out, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);   // n fp32 zeros
hipError_t launch_gather_rows(const void* x, const int32_t* perm, const int32_t* offsets, int n_seg, int k, int d,
                              long long max_rows, void* xg, void* dy, hipStream_t s);
// Tile lists of the grouped GEMM (kind 0: 256- and 64-row tiles, 1: 64-row only, 2: 256-row only).
hipError_t launch_build_tiles(const int32_t* offsets, int n_seg, int dense_rows, int32_t* big, int max_big,
                              int32_t* small, int max_small, int kind, hipStream_t s);
// Backward products with K-major operands (xgemm.hip).
//   NN: out[r, :N] (bf16) = A[r, :K] B_s[K, N] for the rows of segment s; B_s rows k < K1 at
//       B1 + s strideB + k N, rows k >= K1 at B2 + s strideB + (k - K1) N; rows beyond b_rows1 /
//       b_rows2 of either part read as zero.  Needs K, K1 multiples of 64.
//   TN: C_s[m, n] (fp32, row-major [M, N]) = sum over the rows r of segment s of P[r, pc0 + m] Q[r, n].
hipError_t launch_gemm_nn(const void* A, const int32_t* offsets, int n_seg, int dense_rows, int max_rows,
                          int32_t* tiles, int max_tiles, int32_t* tiles_small, int max_tiles_small, const void* B1,
                          const void* B2, long long strideB, int K, int K1, int b_rows1, int b_rows2, int N, void* out,
                          hipStream_t s);
hipError_t launch_gemm_tn(const void* P, int ldp, int pc0, const void* Q, int ldq, const int32_t* offsets, int n_seg,
                          int dense_rows, int max_seg_rows, int M, int N, float* C, long long strideC, hipStream_t s);
hipError_t launch_router_backward(const moe_config& c, const float* z, const int32_t* idx, const float* gates,
                                  const float* dg, const int32_t* counts, float d_aux, float* dz, void* dz16,
                                  int ldz, hipStream_t s);
hipError_t launch_dx_gather(const moe_config& c, const void* dout, const void* dX, const int32_t* slot_pos,
                            const void* dxs, const void* dxr, void* dx, hipStream_t s);

// Top-1 routing with the combine fused into the down projection: the tokens that
// kept no slot get out = [residual] + [shared_y] here.
hipError_t launch_combine_dropped(const moe_config& c, const int32_t* slot_pos, const void* residual,
                                  const void* shared_y, void* out, hipStream_t s);
hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* slot_pos,
                          const float* gates, const void* residual, const void* shared_y,
                          void* out, hipStream_t s);
hipError_t launch_bias_update(const moe_config& c, const int32_t* counts, float gamma,
                              const float* sel_bias_in, float* sel_bias_out, int8_t* signs,
                              hipStream_t s);
hipError_t launch_aux_loss(const moe_config& c, const int32_t* counts, const float* probsum,
                           float* aux, hipStream_t s);

}  // namespace moe
