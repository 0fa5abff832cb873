// Grouped expert GEMM over ragged per-expert row segments.
//
// [L] "Concept / FFN swap": every expert is an independent feed-forward
// network, usually SwiGLU; [G] "How an MoE layer works": experts share one
// architecture; [X] "Future of expert parallelism": grouped GEMMs that batch
// many experts in one launch, and dispatch fused into the expert compute.
// Rows [offsets[e], offsets[e+1]) of the expert-sorted activations go through
// expert e.  With a row permutation (`perm`, slot ids in expert order), the
// up-projection reads those rows straight from the token matrix instead of a
// gathered copy.
//
// Work decomposition.  Every workgroup turns `offsets` into a per-segment
// tile table in LDS (256-row tiles for long segments, 64-row tiles for short
// segments; a long segment's short tail rides on its whole 256-row tiles as
// up to 32 attached rows each, or goes to 64-row tiles; SegTable in
// gemm_tile.h), so the host never waits for the routing result and no launch
// has to write a tile list first.  Two
// persistent kernels run, one per tile kind: the 256-row tiles are bound by
// the matrix cores and run on 8 wavefronts per CU, the 64-row tiles are bound
// by streaming the expert's weights and run on 4.  A K-split fix-up kernel
// closes the call.
//
// MFMA 32x32x16 layout (lane l): A row l%32, k = 8*(l/32)..+7; B column l%32,
// same k; D column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#include <type_traits>

#include "gemm_tile.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


// Tile lists for the backward's NN product (xgemm.hip): every segment split
// into 256-row and 64-row tiles as SegTable does (kind 0, 1), or into 256-row
// tiles only (kind 2: ceil(rows / 256)).  Each list: [0] = tile count; tile i
// at [4 + 8 i] = (segment, row_begin, row_end, first tile of the segment in
// this list, tiles of the segment in this list, 0, 0, 0).
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets, int n_seg,
                                                          int dense_rows, int32_t* __restrict__ big,
                                                          int max_big, int32_t* __restrict__ small,
                                                          int max_small, int kind) {
  __shared__ int tot_b[4], tot_s[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int lo = 0, hi = 0, nb = 0, ns = 0, split = 0;
  if (tid < n_seg) {
    lo = offsets ? offsets[tid] : 0;
    hi = offsets ? offsets[tid + 1] : dense_rows;
    const int rows = hi - lo;
    nb = kind == 1 ? 0 : (kind == 2 ? (rows + 255) / 256 : rows / 256);
    const int rest = rows - nb * 256;
    if (kind == 0 && rest >= kBigTailMin) { nb += 1; }
    else if (rest > 0) { ns = (rest + 63) / 64; }
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

// Kernel arguments of the bf16 grouped GEMM.
struct GemmParams {
  const uint16_t* A;          // rows in expert order, or (gather) the token rows
  const int32_t* perm;        // gather: expert-order row -> slot id; token = slot / gk
  int gk;                     // gather: slots per token
  uint32_t a_bytes;           // gather: bytes of the token matrix
  const uint16_t* W;          // [n_seg, Nn, K]
  const uint16_t* W3;         // SwiGLU: [n_seg, Nn, K]
  const uint16_t* bias;       // [n_seg, Nn] or null
  const uint8_t* W8;          // fp8 weights [n_seg, Nn, K] (E4M3 codes)
  const uint8_t* W8_3;        // fp8 SwiGLU W3
  const float* scale1;        // fp8 row scales of W8 [n_seg, Nn]
  const float* scale3;        // fp8 row scales of W8_3
  uint16_t* out;              // [rows, Nn]
  uint16_t* pre;              // up modes: pre-activations [n_mat][rows, Nn] (bf16) or null
  CombineOut cmb;             // down mode: fused top-1 combine (cmb.out null: plain Y)
  long long pre_plane;        // elements per plane of `pre`
  float* out_f;               // MODE_LOGITS: fp32 output
  const float* bias_f;        // MODE_LOGITS: fp32 bias [Nn] or null
  float* partials;            // K-part tiles of the 256-row list
  float* partials_small;      // K-part tiles of the 64-row list
  int K, Nn, n_ntiles;
  const int32_t* offsets;     // segment row offsets [n_seg + 1], or null: one dense segment of dense_rows
  int n_seg, dense_rows, kind;   // kind: tile table kind (0: 256- and 64-row tiles, 1: 64-row only)
  int attach;                    // short tails attach to whole 256-row tiles (tile kind 0 becomes 5)
};

template <int MODE, bool HAS_BIAS, int NMI = 2>
__device__ __forceinline__ void store_block64(f32x16 (&acc)[NMI][2], float* ep, int lane, int kh, int l32, int wn,
                                              int r0, int r1, int n0, int Nn, int seg,
                                              const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                                              const float* __restrict__ bias_f, float* __restrict__ out_f,
                                              uint16_t* __restrict__ pre, long long pre_plane,
                                              const CombineOut* cmb) {
#pragma unroll
  for (int mi = 0; mi < NMI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[ep_at((r >> 2) * 8 + kh * 4 + (r & 3), ni * 32 + l32)] = acc[mi][ni][r];
    __builtin_amdgcn_wave_barrier();
    const int rbase = r0 + mi * 32;
    if (MODE == MODE_LOGITS) {
#pragma unroll 1
      for (int pass = 0; pass < 8; ++pass) {
        const int rr = pass * 4 + (lane >> 4), c4 = (lane & 15) * 4;
        const int row = rbase + rr, col = n0 + wn * 64 + c4;
        if (row < r1 && col < Nn) {
          float4 v = *reinterpret_cast<const float4*>(ep + ep_at(rr, c4));
          if (HAS_BIAS) {
            const float4 b = *reinterpret_cast<const float4*>(bias_f + col);
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
          }
          *reinterpret_cast<float4*>(out_f + (size_t)row * Nn + col) = v;
        }
      }
    } else if (MODE == MODE_SWIGLU_UP) {
      // cols 0..31 hold x W1^T, cols 32..63 the matching x W3^T
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) {
        const int rr = pass * 16 + (lane >> 2), c8 = (lane & 3) * 8;
        const int row = rbase + rr, col = n0 + wn * 32 + c8;
        if (row < r1 && col < Nn) {
          float src[40];   // columns c8 .. c8 + 7 and c8 + 32 .. c8 + 39 of the row (only those are read)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = c8 + (q & 1) * 4 + (q >> 1) * 32;
            *reinterpret_cast<float4*>(src + (q & 1) * 4 + (q >> 1) * 32) =
                *reinterpret_cast<const float4*>(ep + ep_at(rr, c));
          }
          float hv[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) hv[v] = silu_f(src[v]) * src[32 + v];
          *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = pack_bf16x8(hv);
          if (pre != nullptr) {
            *reinterpret_cast<uint4*>(pre + (size_t)row * Nn + col) = pack_bf16x8(*reinterpret_cast<float(*)[8]>(src));
            *reinterpret_cast<uint4*>(pre + pre_plane + (size_t)row * Nn + col) =
                pack_bf16x8(*reinterpret_cast<float(*)[8]>(src + 32));
          }
        }
      }
    } else {
#pragma unroll 1
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const int row = rbase + rr, col = n0 + wn * 64 + c8;
        if (row < r1 && col < Nn) {
          float src[8];
#pragma unroll
          for (int q = 0; q < 2; ++q)
            *reinterpret_cast<float4*>(src + q * 4) = *reinterpret_cast<const float4*>(ep + ep_at(rr, c8 + q * 4));
          Vec8 b, o, a;
          if (HAS_BIAS) b.u = *reinterpret_cast<const uint4*>(bias + (size_t)seg * Nn + col);
          float xa[8], xo[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            xa[v] = HAS_BIAS ? src[v] + bf16_to_f32(b.e[v]) : src[v];
            xo[v] = MODE == MODE_GELU_UP ? gelu_f(xa[v]) : xa[v];
          }
          o.u = pack_bf16x8(xo);
          if (MODE == MODE_GELU_UP && pre != nullptr) a.u = pack_bf16x8(xa);
          if (MODE == MODE_DOWN && cmb->out != nullptr) {
            combine_store8(*cmb, row, col, Nn, o);
          } else if (MODE == MODE_DOWN) {
            // Y is written once and read once by the combine: a streaming store
            // (DeepSeek-V3 shapes: down projection 2.87 -> 2.82 ms, shared
            // expert 0.715 -> 0.695 ms; Mixtral unchanged; slower for H)
            __builtin_nontemporal_store(u32x4{o.u.x, o.u.y, o.u.z, o.u.w},
                                        reinterpret_cast<u32x4*>(out + (size_t)row * Nn + col));
          } else {
            *reinterpret_cast<uint4*>(out + (size_t)row * Nn + col) = o.u;
          }
          if (MODE == MODE_GELU_UP && pre != nullptr) *reinterpret_cast<uint4*>(pre + (size_t)row * Nn + col) = a.u;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Epilogue of the attached rows of a 256-row unit: each wavefront stages its
// 32 x 32 fp32 block (rows x0.., the 32 columns of its B block ni = wm) in
// LDS, then the outputs are formed and stored 8 columns per lane.  SwiGLU: the
// W1 block of wavefront wn and the W3 block of wavefront wn + 4 meet there.
template <int MODE, bool HAS_BIAS>
__device__ __forceinline__ void store_attached(const GemmParams& p, const Unit& w, const f32x16& accx, float* xs,
                                               int wave, int lane) {
  const int wm = wave >> 2, wn = wave & 3, l32 = lane & 31, kh = lane >> 5;
  float* mine = xs + wave * 1024;
#pragma unroll
  for (int r = 0; r < 16; ++r) mine[(8 * (r >> 2) + 4 * kh + (r & 3)) * 32 + l32] = accx[r];
  __syncthreads();
  const int nxr = w.x1 - w.x0;
  if (MODE == MODE_SWIGLU_UP) {
    if (wave < 4) {
      const float* a = xs + wn * 1024;
      const float* b = xs + (wn + 4) * 1024;
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) {
        const int rr = pass * 16 + (lane >> 2), c8 = (lane & 3) * 8;
        const int row = w.x0 + rr, col = w.n0 + 32 * wn + c8;
        if (rr < nxr && col < p.Nn) {
          float av[8], bv[8], hv[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            av[v] = a[rr * 32 + c8 + v];
            bv[v] = b[rr * 32 + c8 + v];
            hv[v] = silu_f(av[v]) * bv[v];
          }
          *reinterpret_cast<uint4*>(p.out + (size_t)row * p.Nn + col) = pack_bf16x8(hv);
          if (p.pre != nullptr) {
            *reinterpret_cast<uint4*>(p.pre + (size_t)row * p.Nn + col) = pack_bf16x8(av);
            *reinterpret_cast<uint4*>(p.pre + p.pre_plane + (size_t)row * p.Nn + col) = pack_bf16x8(bv);
          }
        }
      }
    }
  } else if (MODE == MODE_GELU_UP || MODE == MODE_DOWN) {
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int rr = pass * 16 + (lane >> 2), c8 = (lane & 3) * 8;
      const int row = w.x0 + rr, col = w.n0 + 64 * wn + 32 * wm + c8;
      if (rr < nxr && col < p.Nn) {
        Vec8 b, o, a;
        if (HAS_BIAS) b.u = *reinterpret_cast<const uint4*>(p.bias + (size_t)w.seg * p.Nn + col);
        float xa[8], xo[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          xa[v] = HAS_BIAS ? mine[rr * 32 + c8 + v] + bf16_to_f32(b.e[v]) : mine[rr * 32 + c8 + v];
          xo[v] = MODE == MODE_GELU_UP ? gelu_f(xa[v]) : xa[v];
        }
        o.u = pack_bf16x8(xo);
        if (MODE == MODE_GELU_UP && p.pre != nullptr) a.u = pack_bf16x8(xa);
        if (MODE == MODE_DOWN)
          __builtin_nontemporal_store(u32x4{o.u.x, o.u.y, o.u.z, o.u.w},
                                      reinterpret_cast<u32x4*>(p.out + (size_t)row * p.Nn + col));
        else
          *reinterpret_cast<uint4*>(p.out + (size_t)row * p.Nn + col) = o.u;
        if (MODE == MODE_GELU_UP && p.pre != nullptr) *reinterpret_cast<uint4*>(p.pre + (size_t)row * p.Nn + col) = a.u;
      }
    }
  }
}

// Workgroup barrier for LDS hand-offs: this wavefront's LDS operations complete, then s_barrier.
// Unlike __syncthreads() it does not wait for the wavefront's global stores.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  MOE_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Stores 32 staged rows (rows 32q.. of `src`, SC bf16 columns, row pitch RS) of a 256-row unit to
// output rows r0 + rbase + 32q.., 16 bytes per lane.
template <int MODE, int SC, int RS>
__device__ __forceinline__ void store_staged(const GemmParams& p, const Unit& w, const uint16_t* src, int rbase, int q,
                                             int lane) {
  constexpr int LPR = SC / 8, RPI = 64 / LPR, NI = 32 / RPI;   // lanes per row, rows per instruction
  const int c8 = (lane % LPR) * 8, col = w.n0 + c8;
  uint4 v[NI];   // every LDS read first, then the stores (one wait, not one per row)
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = *reinterpret_cast<const uint4*>(src + (32 * q + RPI * i + lane / LPR) * RS + c8);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = w.r0 + rbase + 32 * q + RPI * i + lane / LPR;
    if (row < w.r1 && col < p.Nn) {
      if (MODE == MODE_DOWN)   // Y is read once, by the combine: a streaming store
        __builtin_nontemporal_store(u32x4{v[i].x, v[i].y, v[i].z, v[i].w},
                                    reinterpret_cast<u32x4*>(p.out + (size_t)row * p.Nn + col));
      else
        *reinterpret_cast<uint4*>(p.out + (size_t)row * p.Nn + col) = v[i];
    }
  }
}

// Epilogue of a whole 256-row unit (SwiGLU, GELU or down projection; no K-part, no pre-activation
// copy, no fused combine).  Wavefronts 0-3 issue all operand loads and wavefronts 4-7 all output
// stores, so the stores drain while the next unit computes instead of holding up its first step:
// every wavefront rounds its outputs to bf16 into LDS (tile rows 0..127 into the stage-1 buffer,
// rows 128..255 into stage 0, attached rows into the tail); after a barrier wavefronts 4-7 store
// stage 0's rows, a second barrier hands stage 0 to the next unit's first loads, and they store
// the rest (the next unit writes stage 1 only after its first step's barrier).
template <int MODE, bool HAS_BIAS>
__device__ __forceinline__ void store_split(const GemmParams& p, const Unit& w, const f32x16 (&acc)[4][2],
                                            const f32x16& accx, uint16_t* lds, int wave, int lane) {
  constexpr bool SW = MODE == MODE_SWIGLU_UP;
  constexpr int SC = SW ? kBN2 / 2 : kBN2;   // staged columns per row
  constexpr int RS = SC + 8;                  // pitch: rows r and r + 4 of one write fall on other banks
  asm volatile("" : "+v"(lane));   // the LDS and store addresses are formed here, not kept across the unit
  const int wm = wave >> 2, wn = wave & 3, l32 = lane & 31, kh = lane >> 5;
  const int nxr = w.x1 - w.x0;
  uint16_t* S = lds + (wm ? 0 : kStage2);
  uint16_t* T = lds + kTailOff;
  // accumulator register r of a 32 x 32 block: row 8 (r >> 2) + 4 kh + (r & 3), column l32
  if (SW) {   // W1 and W3 columns of one output sit in one lane (blocks ni = 0 and 1)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = 32 * mi + 8 * (r >> 2) + 4 * kh + (r & 3);
        const uint32_t v = pack_bf16x2(silu_f(acc[mi][0][r]) * acc[mi][1][r],
                                       silu_f(acc[mi][0][r + 1]) * acc[mi][1][r + 1]);
        S[row * RS + 32 * wn + l32] = (uint16_t)v;
        S[(row + 1) * RS + 32 * wn + l32] = (uint16_t)(v >> 16);
      }
    if (nxr > 0 && wm == 0) {   // the attached rows' W1 block, for wavefront wn + 4 (which holds W3)
      float* tw = reinterpret_cast<float*>(T) + wn * 1024;
#pragma unroll
      for (int r = 0; r < 16; ++r) tw[r * 64 + lane] = accx[r];
    }
  } else {
    float b[2] = {0.f, 0.f}, bx = 0.f;
    if (HAS_BIAS) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = w.n0 + 64 * wn + 32 * ni + l32;
        b[ni] = col < p.Nn ? bf16_to_f32(p.bias[(size_t)w.seg * p.Nn + col]) : 0.f;
      }
      bx = b[wm];
    }
    auto act = [&](float x) { return MODE == MODE_GELU_UP ? gelu_f(x) : x; };
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = 32 * mi + 8 * (r >> 2) + 4 * kh + (r & 3);
          const uint32_t v = pack_bf16x2(act(acc[mi][ni][r] + b[ni]), act(acc[mi][ni][r + 1] + b[ni]));
          S[row * RS + 64 * wn + 32 * ni + l32] = (uint16_t)v;
          S[(row + 1) * RS + 64 * wn + 32 * ni + l32] = (uint16_t)(v >> 16);
        }
    if (nxr > 0) {   // attached rows: columns 64 wn + 32 wm + l32
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        const uint32_t v = pack_bf16x2(act(accx[r] + bx), act(accx[r + 1] + bx));
        T[row * RS + 64 * wn + 32 * wm + l32] = (uint16_t)v;
        T[(row + 1) * RS + 64 * wn + 32 * wm + l32] = (uint16_t)(v >> 16);
      }
    }
  }
  lds_barrier();   // the staged tile is complete
  const int q = wave - 4;
  if (wm == 1) store_staged<MODE, SC, RS>(p, w, lds, 128, q, lane);
  lds_barrier();   // stage 0 is free for the next unit's first loads
  if (wm == 1) {
    store_staged<MODE, SC, RS>(p, w, lds + kStage2, 0, q, lane);
    if (nxr > 0) {
      if (SW) {
        float* tw = reinterpret_cast<float*>(T) + q * 1024;
        float hv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) hv[r] = silu_f(tw[r * 64 + lane]) * accx[r];
        asm volatile("" ::: "memory");   // the W1 values are read before this wavefront reuses their slot
        uint16_t* tb = T + q * 2048;      // 32 x 32 bf16, pitch 40
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
          const uint32_t v = pack_bf16x2(hv[r], hv[r + 1]);
          tb[row * 40 + l32] = (uint16_t)v;
          tb[(row + 1) * 40 + l32] = (uint16_t)(v >> 16);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rr = 16 * i + (lane >> 2), c8 = (lane & 3) * 8;
          const int col = w.n0 + 32 * q + c8;
          if (rr < nxr && col < p.Nn)
            *reinterpret_cast<uint4*>(p.out + (size_t)(w.x0 + rr) * p.Nn + col) =
                *reinterpret_cast<const uint4*>(tb + rr * 40 + c8);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 8 * q + 2 * i + (lane >> 5), c8 = (lane & 31) * 8;
          const int col = w.n0 + c8;
          if (rr < nxr && col < p.Nn) {
            const uint4 v = *reinterpret_cast<const uint4*>(T + rr * RS + c8);
            if (MODE == MODE_DOWN)
              __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                          reinterpret_cast<u32x4*>(p.out + (size_t)(w.x0 + rr) * p.Nn + col));
            else
              *reinterpret_cast<uint4*>(p.out + (size_t)(w.x0 + rr) * p.Nn + col) = v;
          }
        }
      }
    }
    MOE_WAIT_LGKM0();   // every read of stage 1 is complete before the next unit's first barrier
  }
}

// ---------------------------------------------------------------------------
// 256 x 256 tile (long segments: the routed experts of prefill batches, the
// shared expert, the router logits).
//
// 512 threads = 8 wavefronts, two per SIMD, in a 2 x 4 layout; each wavefront
// owns a 128 x 64 block = 4 x 2 MFMA 32x32x16 blocks (128 fp32 accumulators
// per lane), so while one wavefront of a SIMD waits on its loads or fragment
// reads the other issues MFMAs; s_setprio favours the wavefront that is in
// its MFMA run.  Two 64 KB LDS stages (A 256 rows, B 256 rows, 128 bytes
// each); wavefronts 0-3 issue the loads for step k+1 in slices between the
// MFMAs of the first two sub-steps of step k, and the fragments of each
// 16-wide sub-step are read from LDS while the previous sub-step's 8 MFMAs
// issue.  One fence-free barrier per step.  Wavefronts 4-7 issue no loads and
// store the whole output tile (store_split), so their stores never stall a
// K step (a load wait counts a wavefront's stores too).
//   SwiGLU up : the B tile holds 128 rows of W1 and the same 128 rows of W3;
//               wavefront wn owns W1 columns 32 wn .. 32 wn + 31 (B rows
//               32 wn + ..) and the same W3 columns (B rows 128 + 32 wn + ..),
//               so the epilogue forms SiLU(a1) * a3 in registers and writes
//               bf16 H.
//   GELU up   : GELU(acc + b1) -> bf16 H.
//   down      : acc (+ b2) -> bf16 Y, or the fused top-1 combine.
//   logits    : acc (+ fp32 bias) -> fp32.
template <int MODE, bool HAS_BIAS, bool GATHER>
__device__ __forceinline__ void big_unit(const GemmParams& p, const Unit& w, uint16_t* lds, int wave, int lane) {
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, kh = lane >> 5;
  const size_t wstride = (size_t)p.Nn * p.K;
  const int rowbytes = p.K * 2;
  constexpr bool SW = MODE == MODE_SWIGLU_UP;
  constexpr int cols_per_tile = SW ? kBN2 / 2 : kBN2;

  // DMA: wavefronts 0-3 fill the stages, wavefront w rows 64w .. 64w + 63 of both operands, 8 rows per
  // instruction; wavefronts 4-7 issue no loads, so none of their K steps waits on their output stores
  // (they store every output, see store_split).  Row 64w + 8u + (lane >> 3) takes 16-byte chunk c0 ^ u
  // of its K slice (c0 = (lane & 7) ^ (lane >> 3), the swizzle of swz8), so its offset is that of u = 0
  // with the chunk bits flipped and 8u rows added (row pitches are multiples of 128 bytes).
  const bool dmaw = wave < 4;
  const int l8 = lane >> 3, c0 = (lane & 7) ^ l8;
  const int arow0 = 64 * (wave & 3) + l8;
  int va0 = arow0 * rowbytes + (c0 << 4);
  int vb0 = (SW ? (arow0 & 127) : arow0) * rowbytes + (c0 << 4);   // SwiGLU: W1 rows, then the W3 rows
  int vg[8];
  if (GATHER && dmaw) {   // the 8 token indices are loaded back to back (rows past the tile read its last one)
    int pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pv[u] = p.perm[min(w.r0 + arow0 + 8 * u, w.r1 - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      vg[u] = (w.r0 + arow0 + 8 * u < w.r1 && pv[u] >= 0 ? (pv[u] / p.gk) * rowbytes : kOobOffset) + ((c0 ^ u) << 4);
  }
  // Fragment reads: A rows wm 128 + 32 mi + l32 -> slot (2 kk + kh) ^ g(l32) ^ 4 (mi & 1);
  // B rows (SwiGLU) 128 ni + 32 wn + l32 -> ^ 4 (wn & 1), else 64 wn + 32 ni + l32 -> ^ 4 (ni & 1).
  const int h = kh ^ swz8(l32);
  const int abase = (wm * 128 + l32) * kBK2;
  const int bb0 = kStageA + (SW ? (32 * wn + l32) : (64 * wn + l32)) * kBK2;
  const int bstep = (SW ? 128 : 32) * kBK2;
  const int hb0 = SW ? (h ^ (4 * (wn & 1))) : h;
  const int hb1 = SW ? hb0 : (h ^ 4);

  const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(p.A, p.a_bytes)
                                           : make_rsrc(p.A + (size_t)w.r0 * p.K, (uint32_t)(w.r1 - w.r0) * rowbytes);
  const int nb_rows = min(cols_per_tile, p.Nn - w.n0);
  const uint16_t* wsrc = (SW && wave >= 2) ? p.W3 : p.W;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(wsrc + (size_t)w.seg * wstride + (size_t)w.n0 * p.K, (uint32_t)nb_rows * rowbytes);
  auto aoff = [&](int u) { return GATHER ? vg[u] : (va0 ^ (u << 4)) + u * 8 * rowbytes; };
  auto boff = [&](int u) { return (vb0 ^ (u << 4)) + u * 8 * rowbytes; };

  // attached tail rows [x0, x1): A rows 256 .. 287 of the stage, loaded by wavefronts 0-3 (8 rows each);
  // wavefront (wm, wn) multiplies them by its B block ni = wm (32 columns)
  const int nxr = w.x1 - w.x0;
  int voffx = kOobOffset;
  __amdgpu_buffer_rsrc_t rax = ra;
  if (nxr > 0 && dmaw) {
    const int row = 8 * (wave & 3) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);   // swz8(256 + row) = swz8(row)
    if (GATHER) {
      const int r = w.x0 + row;
      const int pr = r < w.x1 ? p.perm[r] : -1;
      voffx = (pr >= 0 ? (pr / p.gk) * rowbytes : kOobOffset) + chunk * 16;
    } else {
      rax = make_rsrc(p.A + (size_t)w.x0 * p.K, (uint32_t)nxr * rowbytes);
      voffx = row * rowbytes + chunk * 16;
    }
  }
  const bool xload = nxr > 0 && wave < 4;
  f32x16 acc[4][2], accx;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) accx[r] = 0.f;

  const int kt0 = w.kt0, kt1 = w.kt1;
  // the ring counts from the unit's first step: that step's loads go to stage 0 (store_split keeps
  // stage 1 busy into the next unit)
  if (kt0 < kt1 && dmaw) {
    const int so = kt0 * kBK2 * 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dma16(ra, lds + (64 * wave + 8 * u) * kBK2, aoff(u), so);
      dma16(rb, lds + kStageA + (64 * wave + 8 * u) * kBK2, boff(u), so);
    }
    if (xload) dma16(rax, lds + (256 + 8 * wave) * kBK2, voffx, so);
  }
  // live 32-row blocks of this wavefront: a tile that ends inside the wavefront's 128 rows
  // (the tail of a long segment) skips the MFMAs and fragment reads of the empty blocks
  const int nv = __builtin_amdgcn_readfirstlane(min(4, max(0, (w.r1 - w.r0 - wm * 128 + 31) / 32)));
  auto step = [&](const uint16_t* __restrict__ st, uint16_t* __restrict__ nx, int kt, auto nv_t) {
    constexpr int NV = decltype(nv_t)::value;
    if (dmaw) MOE_WAIT_VM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" : "+v"(va0), "+v"(vb0));   // the 16 offsets are formed per load, not kept in registers
    const bool more = kt + 1 < kt1;
    const int so = (kt + 1) * kBK2 * 2;
    bf16x8 fa[2][4], fb[2][2];
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (x < NV) fa[0][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + ((h ^ (4 * (x & 1))) << 3));
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (NV > 0) fb[0][x] = *reinterpret_cast<const bf16x8*>(st + bb0 + bstep * x + ((x ? hb1 : hb0) << 3));
#pragma unroll
    for (int kk = 0; kk < kBK2 / 16; ++kk) {
      const int c = kk & 1;
      if (more && kk < 2 && dmaw) {
#pragma unroll
        for (int u = 4 * kk; u < 4 * kk + 4; ++u) {
          dma16(ra, nx + (64 * wave + 8 * u) * kBK2, aoff(u), so);
          dma16(rb, nx + kStageA + (64 * wave + 8 * u) * kBK2, boff(u), so);
        }
      }
      if (kk + 1 < kBK2 / 16) {
        const int k2 = 2 * (kk + 1);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x < NV)
            fa[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + ((h ^ (4 * (x & 1)) ^ k2) << 3));
#pragma unroll
        for (int x = 0; x < 2; ++x)
          if (NV > 0)
            fb[c ^ 1][x] = *reinterpret_cast<const bf16x8*>(st + bb0 + bstep * x + (((x ? hb1 : hb0) ^ k2) << 3));
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mi = 0; mi < NV; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      if (NV == 4) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);   // 3 MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
  };
  // A whole tile with attached rows: the A fragments are read at the start of each sub-step
  // instead of one ahead (the registers go to the attached rows' accumulators), and every
  // wavefront adds one MFMA for the attached rows against its B block ni = wm.
  auto step_x = [&](const uint16_t* __restrict__ st, uint16_t* __restrict__ nx, int kt, auto wm_t) {
    constexpr int WM = decltype(wm_t)::value;   // = wm: the B block the attached rows use
    if (dmaw) MOE_WAIT_VM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" : "+v"(va0), "+v"(vb0));   // the 16 offsets are formed per load, not kept in registers
    const bool more = kt + 1 < kt1;
    const int so = (kt + 1) * kBK2 * 2;
    bf16x8 fb[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
      fb[0][x] = *reinterpret_cast<const bf16x8*>(st + bb0 + bstep * x + ((x ? hb1 : hb0) << 3));
#pragma unroll
    for (int kk = 0; kk < kBK2 / 16; ++kk) {
      const int c = kk & 1, k2 = 2 * kk;
      if (more && kk < 2 && dmaw) {
#pragma unroll
        for (int u = 4 * kk; u < 4 * kk + 4; ++u) {
          dma16(ra, nx + (64 * wave + 8 * u) * kBK2, aoff(u), so);
          dma16(rb, nx + kStageA + (64 * wave + 8 * u) * kBK2, boff(u), so);
        }
        if (kk == 1 && xload) dma16(rax, nx + (256 + 8 * wave) * kBK2, voffx, so);
      }
      bf16x8 fa[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        fa[x] = *reinterpret_cast<const bf16x8*>(st + abase + 2048 * x + ((h ^ (4 * (x & 1)) ^ k2) << 3));
      const bf16x8 fx = *reinterpret_cast<const bf16x8*>(st + (256 + l32) * kBK2 + ((h ^ k2) << 3));
      if (kk + 1 < kBK2 / 16) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
          fb[c ^ 1][x] =
              *reinterpret_cast<const bf16x8*>(st + bb0 + bstep * x + (((x ? hb1 : hb0) ^ (k2 + 2)) << 3));
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
      accx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx, fb[c][WM], accx, 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  };
  auto loop = [&](auto nv_t) {
    for (int kt = kt0; kt < kt1; ++kt)
      step(lds + ((kt - kt0) & 1) * kStage2, lds + ((kt - kt0 + 1) & 1) * kStage2, kt, nv_t);
  };
  if (nxr > 0) {   // attached rows come only with whole 256-row tiles
    auto loop_x = [&](auto wm_t) {
      for (int kt = kt0; kt < kt1; ++kt)
        step_x(lds + ((kt - kt0) & 1) * kStage2, lds + ((kt - kt0 + 1) & 1) * kStage2, kt, wm_t);
    };
    if (wm) loop_x(std::integral_constant<int, 1>{});
    else loop_x(std::integral_constant<int, 0>{});
  } else
  switch (nv) {
    case 4: loop(std::integral_constant<int, 4>{}); break;
    case 3: loop(std::integral_constant<int, 3>{}); break;
    case 2: loop(std::integral_constant<int, 2>{}); break;
    case 1: loop(std::integral_constant<int, 1>{}); break;
    default: loop(std::integral_constant<int, 0>{}); break;
  }
  // Nothing is in flight here but the previous unit's output stores of wavefronts 4-7, long done;
  // the wait also tells the compiler that no direct-to-LDS load is, so the epilogue's LDS reads
  // need no wait of their own (a wait would also wait for the stores issued just before them).
  MOE_WAIT_VM0();
  lds_barrier();   // every wavefront is done with the ring

  constexpr bool SPLIT = MODE == MODE_SWIGLU_UP || MODE == MODE_GELU_UP || MODE == MODE_DOWN;
  if (SPLIT && w.slot < 0 && p.pre == nullptr && p.cmb.out == nullptr) {
    store_split<MODE, HAS_BIAS>(p, w, acc, accx, lds, wave, lane);
  } else if (w.slot < 0) {
    float* ep = reinterpret_cast<float*>(lds) + wave * (32 * 64);
    store_block64<MODE, HAS_BIAS, 4>(acc, ep, lane, kh, l32, wn, w.r0 + wm * 128, w.r1, w.n0, p.Nn, w.seg, p.bias,
                                     p.out, p.bias_f, p.out_f, p.pre, p.pre_plane, &p.cmb);
    if (nxr > 0) store_attached<MODE, HAS_BIAS>(p, w, accx, reinterpret_cast<float*>(lds) + 16384, wave, lane);
    __syncthreads();   // the next unit's first loads must not overtake this epilogue
  } else {
    // fp32 partial tile, row-major [slot][kBM2P rows][256 accumulator columns] (rows 256 .. 287: the
    // attached rows); SwiGLU holds W1 and W3 columns in blocks of 64 (the K-part fix-up reads that layout)
    float* dst = p.partials + (size_t)w.slot * (kBM2P * kBN2) + (size_t)(wm * 128 + 4 * kh) * kBN2;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      int col;
      if (SW) {
        const int j = 32 * wn + l32;                      // W1 / W3 output column of this lane
        col = (j >> 6) * 128 + (j & 63) + 64 * ni;
      } else {
        col = 64 * wn + 32 * ni + l32;
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(mi * 32 + 8 * (r >> 2) + (r & 3)) * kBN2 + col] = acc[mi][ni][r];
    }
    if (nxr > 0) {
      int col;
      if (SW) {
        const int j = 32 * wn + l32;
        col = (j >> 6) * 128 + (j & 63) + 64 * wm;
      } else {
        col = 64 * wn + 32 * wm + l32;
      }
      float* dx = p.partials + (size_t)w.slot * (kBM2P * kBN2) + (size_t)(256 + 4 * kh) * kBN2 + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) dx[(8 * (r >> 2) + (r & 3)) * kBN2] = accx[r];
    }
  }
}

// Persistent over the 256-row tile list: the grid holds one workgroup per CU,
// XCD-major (workgroup b runs on XCD b % 8), and each XCD takes a contiguous
// span of the whole (tile, column tile) units, so that the units sharing an
// expert's weights meet in one L2, and one of the K-part units (xcd_slice).
template <int MODE, bool HAS_BIAS, bool GATHER>
__global__ __launch_bounds__(512, 1) void grouped_gemm_big_kernel(GemmParams p) {
  // one LDS object: the operand stages, then the tile table (a second __shared__ object
  // would keep the compiler from telling the fragment reads apart from the in-flight
  // direct-to-LDS loads, and it would then wait for those loads before every read)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kTailOff + kTailElems];
  SegTable& segt = *reinterpret_cast<SegTable*>(lds + 2 * kStage2);
  static_assert(2 * kStage2 * 2 >= 96 * 1024, "the epilogue staging (64 KB + 32 KB of attached rows) fits the ring");
  static_assert(128 * (kBN2 + 8) <= kStage2, "store_split stages 128 rows of the tile in one operand stage");
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int G = gridDim.x;
  const int KT = p.K / kBK2;
  build_seg_table(segt, p.offsets, p.n_seg, p.dense_rows, p.kind, p.n_ntiles, G, p.attach != 0);
  const UnitPlan pb = plan_units(segt.pb[p.n_seg] * p.n_ntiles, G, KT);
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  const XcdSlice xs = xcd_slice(pb, xcd);
  const int cb = xs.fc + xs.pc;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  for (int i = q; i < cb; i += per_xcd) {
    const Unit w = decode_unit_lds(segt, p.n_seg, true, pb, xcd_unit(pb, xs, i), p.n_ntiles, KT, cols_per_tile);
    big_unit<MODE, HAS_BIAS, GATHER>(p, w, lds, wave, lane);
  }
}

// ---------------------------------------------------------------------------
// 64 x 256 tile (short segments: decode batches, experts with few routed
// rows, the short tails of long segments).  There the GEMM streams the
// expert's weights for a handful of rows, so the design goal is many bytes in
// flight per CU rather than MFMA reuse: 4 wavefronts in a 1 x 4 layout, each
// 64 x 64 (2 x 2 MFMA 32x32x16 blocks), and a 3-stage LDS ring of 40 KB stages
// (A: 64 rows, B: 256 rows, 128 bytes each) keeps two K steps of loads in
// flight.  The weights, read once per call, arrive as nontemporal loads.
template <int MODE, bool HAS_BIAS, bool GATHER>
__device__ __forceinline__ void small_unit(const GemmParams& p, const Unit& w, uint16_t* lds, int wn, int lane) {
  const int l32 = lane & 31, kh = lane >> 5;
  const size_t wstride = (size_t)p.Nn * p.K;
  const int rowbytes = p.K * 2;
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;

  // DMA: wavefront w fills A rows 16w..16w+15 (2 instructions) and B rows 64w..64w+63 (8).
  int voffa[2], voffb[8];
  int pv[2];   // gather: the two token indices loaded back to back (rows past the tile read its last one)
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (GATHER) pv[u] = p.perm[min(w.r0 + 16 * wn + 8 * u + (lane >> 3), w.r1 - 1)];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * wn + 8 * u + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);
    if (GATHER) {
      const int pr = w.r0 + row < w.r1 ? pv[u] : -1;   // -1 also: a padding row of the [E, C] layout
      voffa[u] = (pr >= 0 ? (pr / p.gk) * rowbytes : kOobOffset) + chunk * 16;
    } else {
      voffa[u] = row * rowbytes + chunk * 16;
    }
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

  const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(p.A, p.a_bytes)
                                           : make_rsrc(p.A + (size_t)w.r0 * p.K, (uint32_t)(w.r1 - w.r0) * rowbytes);
  const int nb_rows = min(cols_per_tile, p.Nn - w.n0);
  const uint16_t* wsrc = (MODE == MODE_SWIGLU_UP && wn >= 2) ? p.W3 : p.W;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(wsrc + (size_t)w.seg * wstride + (size_t)w.n0 * p.K, (uint32_t)nb_rows * rowbytes);

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int kt0 = w.kt0, kt1 = w.kt1;
  // prologue: steps kt0 and kt0 + 1
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int kt = kt0 + pp;
    if (kt < kt1) {
      uint16_t* st = lds + (kt % kStages3) * kStage3Elems;
      const int so = kt * kBK2 * 2;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) dma16(ra, st + (16 * wn + 8 * uu) * kBK2, voffa[uu], so);
#pragma unroll
      for (int uu = 0; uu < 8; ++uu) dma16_stream(rb, st + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
    }
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    // outstanding in issue order: step kt, then step kt + 1 (10 loads) if it exists
    if (kt + 1 < kt1) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(10));
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
          for (int uu = 0; uu < 2; ++uu) dma16_stream(rb, nx + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
        } else {
#pragma unroll
          for (int uu = 3 * kk - 1; uu < 3 * kk + 2; ++uu)
            dma16_stream(rb, nx + (kBM3 + 64 * wn + 8 * uu) * kBK2, voffb[uu], so);
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

  if (w.slot < 0) {
    float* ep = reinterpret_cast<float*>(lds) + wn * (32 * 64);
    store_block64<MODE, HAS_BIAS>(acc, ep, lane, kh, l32, wn, w.r0, w.r1, w.n0, p.Nn, w.seg, p.bias, p.out,
                                  p.bias_f, p.out_f, p.pre, p.pre_plane, &p.cmb);
  } else {
    // fp32 partial tile, row-major [slot][64 rows][256 accumulator columns]; only the tile's rows
    // (the fix-up reads no others; a decode tile has a handful of its 64)
    float* dst = p.partials_small + (size_t)w.slot * (kBM3 * kBN2) + (size_t)(4 * kh) * kBN2 + wn * 64 + l32;
    const int live = w.r1 - w.r0 - 4 * kh;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mi * 32 + 8 * (r >> 2) + (r & 3) < live) dst[(mi * 32 + 8 * (r >> 2) + (r & 3)) * kBN2 + ni * 32] = acc[mi][ni][r];
  }
  __syncthreads();   // the next unit's first loads must not overtake this epilogue
}

// ---------------------------------------------------------------------------
// 64 x 256 tile with fp8 (E4M3) weights ([S]: quantised expert weights halve
// the bytes a weight-streaming GEMM moves).  The B tile arrives as codes
// through the same direct-to-LDS loads, 128 K per step: every weight row
// contributes one whole 128-byte line per step, so the weight stream moves
// the same line-sized pieces as the bf16 tile (64-K steps, half lines, kept
// the fp8 stream at 4.5 TB/s).  A stage holds the A rows as two 64-K halves
// in the bf16 tile's layout plus 256 B rows of 128 bytes (48 KB); a 3-stage
// ring keeps two steps of loads in flight.  Units keep their K ranges in
// 64-K steps: a unit with an odd count ends with a half step, whose second
// half is loaded as zeros (fp8_a_voff / fp8_b_voff) and not used.  Fragments are
// expanded to bf16 exactly (every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8 at scale 1 and fed to the bf16 MFMA; each output
// column is multiplied by its weight row's scale before the epilogue.
// B LDS layout: row r holds eight 16-byte chunks, chunk c in slot c ^ g(r),
// as for the bf16 operands.
constexpr int kStages8 = 3;
constexpr int kBK8 = 2 * kBK2;                                   // K per fp8 step
constexpr int kStage8A = 2 * kBM3 * kBK2;                        // two 64-K halves of 64 bf16 rows
constexpr int kStage8Elems = kStage8A + (kBN2 * kBK8) / 2;      // + 256 fp8 rows of 128 bytes, in bf16 units
static_assert(kStages8 * kStage8Elems * 2 <= 160 * 1024, "fp8 ring exceeds the CU's LDS");

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 v) {
  union {
    bf16x2v h[4];
    bf16x8 o;
  } u;
  u.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  u.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  u.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  u.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return u.o;
}

// NMI: 32-row MFMA blocks computed (1 when the unit has at most 32 rows, as
// at decode batch sizes; the second block's accumulators then stay zero).
template <int MODE, bool HAS_BIAS, bool GATHER, int NMI>
__device__ __forceinline__ void small_unit_fp8(const GemmParams& p, const Unit& w, uint16_t* lds, int wn,
                                               int lane) {
  constexpr int kLoads = 12;                 // per wavefront and step: 4 A (2 per half) + 8 B
  const int l32 = lane & 31, kh = lane >> 5;
  const int rowbytes = p.K * 2;
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;

  int voffa[2], voffb[8];
  int pv[2];   // gather: the two token indices loaded back to back (rows past the tile read its last one)
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (GATHER) pv[u] = p.perm[min(w.r0 + 16 * wn + 8 * u + (lane >> 3), w.r1 - 1)];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * wn + 8 * u + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);
    if (GATHER) {
      const int pr = w.r0 + row < w.r1 ? pv[u] : -1;   // -1 also: a padding row of the [E, C] layout
      voffa[u] = (pr >= 0 ? (pr / p.gk) * rowbytes : kOobOffset) + chunk * 16;
    } else {
      voffa[u] = row * rowbytes + chunk * 16;
    }
  }
  // B: instruction u of wavefront wn fills rows 64 wn + 8 u + (lane >> 3), slot lane & 7
  // with the row's 16-byte chunk (lane & 7) ^ g(row); voffh[u]: the same on a half step
  int voffh[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 64 * wn + 8 * u + (lane >> 3);
    const int chunk = (lane & 7) ^ swz8(row);
    voffb[u] = (MODE == MODE_SWIGLU_UP ? (row & 127) : row) * p.K + chunk * 16;
    voffh[u] = fp8_b_voff(voffb[u], chunk, true);
  }
  const int h = kh ^ swz8(l32);
  const int brow0 = MODE == MODE_SWIGLU_UP ? (32 * wn + l32) : (64 * wn + l32);
  const int bstep = MODE == MODE_SWIGLU_UP ? 128 : 32;
  // g(row) of the two fragment rows: g(32 m + l32) = g(l32) ^ 4 (m & 1), m = wn + 4 x (SwiGLU) or 2 wn + x
  const int bsw0 = swz8(l32) ^ (MODE == MODE_SWIGLU_UP ? 4 * (wn & 1) : 0);
  const int bsw1 = MODE == MODE_SWIGLU_UP ? bsw0 : (bsw0 ^ 4);

  const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(p.A, p.a_bytes)
                                           : make_rsrc(p.A + (size_t)w.r0 * p.K, (uint32_t)(w.r1 - w.r0) * rowbytes);
  const int nb_rows = min(cols_per_tile, p.Nn - w.n0);
  const uint8_t* wsrc = (MODE == MODE_SWIGLU_UP && wn >= 2) ? p.W8_3 : p.W8;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(wsrc + (size_t)w.seg * p.Nn * p.K + (size_t)w.n0 * p.K, (uint32_t)nb_rows * p.K);

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // per-column weight scales (lane's column l32 of each 32-wide block), loaded before the first
  // operand loads so that their latency is over by the epilogue (the waits below count them too:
  // loads complete in issue order)
  float sc[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int col = MODE == MODE_SWIGLU_UP ? w.n0 + 32 * wn + l32 : w.n0 + 64 * wn + 32 * ni + l32;
    const float* sp = (MODE == MODE_SWIGLU_UP && ni == 1) ? p.scale3 : p.scale1;
    sc[ni] = sp[(size_t)w.seg * p.Nn + min(col, p.Nn - 1)];
    if (col >= p.Nn) sc[ni] = 0.f;
  }
  // step j covers the 64-K steps kt0 + 2j and kt0 + 2j + 1 (the second only if < kt1)
  const int kt0 = w.kt0, n64 = w.kt1 - w.kt0, nst = (n64 + 1) >> 1;
  // loads of step j (k64 = kt0 + 2 j); `half`: step j is a half step (its second 64 K read as zero)
#define FP8_LOAD_A(hf, u, st, k64, half)                                                           \
  dma16(ra, (st) + (hf) * (kBM3 * kBK2) + (16 * wn + 8 * (u)) * kBK2, fp8_a_voff(voffa[u], hf, half), \
        ((k64) + (hf)) * kBK2 * 2)
#define FP8_LOAD_B(u, st, k64, half) \
  dma16(rb, (st) + kStage8A + (64 * wn + 8 * (u)) * (kBK8 / 2), (half) ? voffh[u] : voffb[u], (k64) * kBK2)
#pragma unroll
  for (int pp = 0; pp < kStages8 - 1; ++pp) {   // prologue: steps 0 and 1
    if (pp < nst) {
      uint16_t* st = lds + pp * kStage8Elems;
      const int k64 = kt0 + 2 * pp;
      const bool half = 2 * pp + 1 >= n64;
      FP8_LOAD_A(0, 0, st, k64, half); FP8_LOAD_A(0, 1, st, k64, half);
      FP8_LOAD_A(1, 0, st, k64, half); FP8_LOAD_A(1, 1, st, k64, half);
#pragma unroll
      for (int u = 0; u < 8; ++u) FP8_LOAD_B(u, st, k64, half);
    }
  }
  for (int j = 0; j < nst; ++j) {
    // outstanding loads in issue order: step j, then step j + 1 (kLoads) if it exists
    if (j + 1 < nst) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(kLoads));
    else MOE_WAIT_VM0();
    __builtin_amdgcn_s_barrier();            // step j landed everywhere; the slot of j - 1 is free
    const uint16_t* st = lds + (j % kStages8) * kStage8Elems;
    uint16_t* nx = lds + ((j + 2) % kStages8) * kStage8Elems;
    const bool more = j + 2 < nst;
    const int knx = kt0 + 2 * (j + 2);
    const bool nhalf = 2 * (j + 2) + 1 >= n64;
    const int nsub = 2 * j + 1 < n64 ? 8 : 4;   // a half step computes its first 64 K only
    // fragments of sub-step kk into buffer c: A as read, B's 8 code bytes converted to bf16; the
    // next sub-step's are read and converted while this one's MFMAs issue (with one wavefront
    // per SIMD nothing else would cover the LDS latency and the conversions)
    bf16x8 fa[2][2], fb[2][2];
    auto frag = [&](int kk, int c) {
      const int hf = kk >> 2, kq = kk & 3;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x < NMI)
          fa[c][x] = *reinterpret_cast<const bf16x8*>(st + hf * (kBM3 * kBK2) + (32 * x + l32) * kBK2 +
                                                      ((h ^ (4 * x) ^ (2 * kq)) << 3));
        const int brow = brow0 + bstep * x;
        // 8 code bytes read with the same element type as the A fragments (the compiler then
        // keeps them apart from the in-flight LDS loads as it does for A)
        const bf16x4 b4 = *reinterpret_cast<const bf16x4*>(
            st + kStage8A + ((brow * kBK8 + ((kk ^ (x ? bsw1 : bsw0)) << 4) + kh * 8) >> 1));
        fb[c][x] = fp8x8_to_bf16(__builtin_bit_cast(uint2, b4));
      }
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK8 / 16; ++kk) {
      const int c = kk & 1;
      if (more && kk < 5) {                   // next loads: 4 A, then 2 B in each of the next four sub-steps
        if (kk == 0) {
          FP8_LOAD_A(0, 0, nx, knx, nhalf); FP8_LOAD_A(0, 1, nx, knx, nhalf);
          FP8_LOAD_A(1, 0, nx, knx, nhalf); FP8_LOAD_A(1, 1, nx, knx, nhalf);
        } else {
          FP8_LOAD_B(2 * kk - 2, nx, knx, nhalf); FP8_LOAD_B(2 * kk - 1, nx, knx, nhalf);
        }
      }
      if (kk >= nsub) continue;
      if (kk + 1 < nsub) frag(kk + 1, c ^ 1);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][mi], fb[c][ni], acc[mi][ni], 0, 0, 0);
    }
  }
#undef FP8_LOAD_A
#undef FP8_LOAD_B
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] *= sc[ni];
  __syncthreads();   // every wavefront is done with the ring before the epilogue reuses it

  if (w.slot < 0) {
    float* ep = reinterpret_cast<float*>(lds) + wn * (32 * 64);
    store_block64<MODE, HAS_BIAS>(acc, ep, lane, kh, l32, wn, w.r0, w.r1, w.n0, p.Nn, w.seg, p.bias, p.out,
                                  p.bias_f, p.out_f, p.pre, p.pre_plane, &p.cmb);
  } else {
    float* dst = p.partials_small + (size_t)w.slot * (kBM3 * kBN2) + (size_t)(4 * kh) * kBN2 + wn * 64 + l32;
    const int live = w.r1 - w.r0 - 4 * kh;   // the tile's rows only, as in small_unit
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mi * 32 + 8 * (r >> 2) + (r & 3) < live) dst[(mi * 32 + 8 * (r >> 2) + (r & 3)) * kBN2 + ni * 32] = acc[mi][ni][r];
  }
  __syncthreads();   // the next unit's first loads must not overtake this epilogue
}

// Persistent over the 64-row tile list, same XCD-major unit spans as the
// 256-row kernel.  It runs after the 256-row kernel on the same stream: the
// two tiles want different workgroup shapes (8 and 4 wavefronts).  The pair
// of launches measured faster than the earlier single kernel that ran both
// lists, 256-row units first, with a 4-wavefront 256-row tile.
template <int MODE, bool HAS_BIAS, bool GATHER, bool FP8>
__global__ __launch_bounds__(256, 1) void grouped_gemm_small_kernel(GemmParams p) {
  constexpr int kRing = FP8 ? kStages8 * kStage8Elems : kStages3 * kStage3Elems;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kRing + kSegTableElems];   // one LDS object, as above
  SegTable& segt = *reinterpret_cast<SegTable*>(lds + kRing);
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  const int G = gridDim.x;
  const int KT = p.K / kBK2;
  build_seg_table(segt, p.offsets, p.n_seg, p.dense_rows, p.kind, p.n_ntiles, G, p.attach != 0);
  const UnitPlan ps = plan_units(segt.ps[p.n_seg] * p.n_ntiles, G, KT);
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  const XcdSlice xs = xcd_slice(ps, xcd);
  const int cs = xs.fc + xs.pc;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps buffer descriptors scalar
  const int lane = tid & 63;
  for (int i = q; i < cs; i += per_xcd) {
    const Unit w = decode_unit_lds(segt, p.n_seg, false, ps, xcd_unit(ps, xs, i), p.n_ntiles, KT, cols_per_tile);
    if (FP8) {
      if (w.r1 - w.r0 <= 32) small_unit_fp8<MODE, HAS_BIAS, GATHER, 1>(p, w, lds, wave, lane);
      else small_unit_fp8<MODE, HAS_BIAS, GATHER, 2>(p, w, lds, wave, lane);
    }
    else small_unit<MODE, HAS_BIAS, GATHER>(p, w, lds, wave, lane);
  }
}

// Adds the K-parts of each split tile in part order and runs the epilogue.
// Row-parallel: one thread per (split tile, row, 8 output columns), grid-stride
// over the split tiles of both lists, 16-byte loads and stores.  Accumulator
// column of output column oc: oc itself, except for SwiGLU, where the tile
// holds W1 and W3 columns in blocks of `half` (64 for 256-row tiles, 32 for
// 64-row tiles): a1 = oc + (oc / half) * half, a3 = a1 + half.
template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256) void split_fixup_kernel(GemmParams p, int G) {
  __shared__ SegTable segt;
  constexpr int cols_per_tile = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  constexpr int groups = cols_per_tile / 8;
  const int KT = p.K / kBK2;
  build_seg_table(segt, p.offsets, p.n_seg, p.dense_rows, p.kind, p.n_ntiles, G, p.attach != 0);
  const UnitPlan pb = plan_units(segt.pb[p.n_seg] * p.n_ntiles, G, KT);
  const UnitPlan ps = plan_units(segt.ps[p.n_seg] * p.n_ntiles, G, KT);
  const long long nb = (long long)pb.rem * kBM2P * groups;
  const long long n = nb + (long long)ps.rem * kBM3 * groups;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < n;
       it += (long long)gridDim.x * blockDim.x) {
    const bool big = it < nb;
    const long long jt = big ? it : it - nb;
    const int bm = big ? kBM2P : kBM3;
    const int t = (int)(jt / ((long long)bm * groups));
    const int rem_it = (int)(jt - (long long)t * bm * groups);
    const int row_in = rem_it / groups, oc = (rem_it % groups) * 8;
    const UnitPlan& pl = big ? pb : ps;
    const Unit w = decode_unit_seg(segt, p.n_seg, big, pl, pl.full + t * pl.s, p.n_ntiles, KT, cols_per_tile);
    // partial rows 0 .. 255: the tile's rows; 256 .. 287 (256-row tiles): its attached rows
    const int row = row_in < 256 ? w.r0 + row_in : w.x0 + (row_in - 256);
    const int col = w.n0 + oc;
    if (row >= (row_in < 256 ? w.r1 : w.x1) || col >= p.Nn) continue;
    const float* part = (big ? p.partials : p.partials_small) + (size_t)t * pl.s * bm * kBN2 +
                        (size_t)row_in * kBN2;
    const int half = big ? 64 : 32;
    const int a1 = MODE == MODE_SWIGLU_UP ? oc + (oc / half) * half : oc;
    float v1[8], v3[8];
    for (int q = 0; q < pl.s; ++q) {
      const float* src = part + (size_t)q * bm * kBN2;
      const float4 x0 = *reinterpret_cast<const float4*>(src + a1);
      const float4 x1 = *reinterpret_cast<const float4*>(src + a1 + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v1[e] = q == 0 ? xs[e] : v1[e] + xs[e];
      if (MODE == MODE_SWIGLU_UP) {
        const float4 y0 = *reinterpret_cast<const float4*>(src + a1 + half);
        const float4 y1 = *reinterpret_cast<const float4*>(src + a1 + half + 4);
        const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v3[e] = q == 0 ? ys[e] : v3[e] + ys[e];
      }
    }
    if (MODE == MODE_LOGITS) {
      float4 o0 = make_float4(v1[0], v1[1], v1[2], v1[3]), o1 = make_float4(v1[4], v1[5], v1[6], v1[7]);
      if (HAS_BIAS) {
        const float4 b0 = *reinterpret_cast<const float4*>(p.bias_f + col);
        const float4 b1 = *reinterpret_cast<const float4*>(p.bias_f + col + 4);
        o0.x += b0.x; o0.y += b0.y; o0.z += b0.z; o0.w += b0.w;
        o1.x += b1.x; o1.y += b1.y; o1.z += b1.z; o1.w += b1.w;
      }
      *reinterpret_cast<float4*>(p.out_f + (size_t)row * p.Nn + col) = o0;
      *reinterpret_cast<float4*>(p.out_f + (size_t)row * p.Nn + col + 4) = o1;
      continue;
    }
    Vec8 b, o, s1, s3;
    if (HAS_BIAS) b.u = *reinterpret_cast<const uint4*>(p.bias + (size_t)w.seg * p.Nn + col);
    float xa[8], xo[8];   // the pre-activation (W1 part for SwiGLU) and the output
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (MODE == MODE_SWIGLU_UP) {
        xa[e] = v1[e];
        xo[e] = silu_f(v1[e]) * v3[e];
      } else {
        xa[e] = HAS_BIAS ? v1[e] + bf16_to_f32(b.e[e]) : v1[e];
        xo[e] = MODE == MODE_GELU_UP ? gelu_f(xa[e]) : xa[e];
      }
    }
    o.u = pack_bf16x8(xo);
    s1.u = pack_bf16x8(xa);
    if (MODE == MODE_SWIGLU_UP) s3.u = pack_bf16x8(v3);
    if (MODE == MODE_DOWN && p.cmb.out != nullptr) combine_store8(p.cmb, row, col, p.Nn, o);
    else *reinterpret_cast<uint4*>(p.out + (size_t)row * p.Nn + col) = o.u;
    if ((MODE == MODE_SWIGLU_UP || MODE == MODE_GELU_UP) && p.pre != nullptr) {
      *reinterpret_cast<uint4*>(p.pre + (size_t)row * p.Nn + col) = s1.u;
      if (MODE == MODE_SWIGLU_UP) *reinterpret_cast<uint4*>(p.pre + p.pre_plane + (size_t)row * p.Nn + col) = s3.u;
    }
  }
}

// fp32 storage: one thread per output element, sequential fp32 FMA over K.
// With `perm`, row r of the expert order reads token row perm[r] / gk of A
// (perm[r] = -1: a padding row, all zeros).
template <int MODE, bool HAS_BIAS>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ perm, int gk, const int32_t* __restrict__ offsets,
    int n_seg, int dense_rows, const float* __restrict__ W, const float* __restrict__ W3,
    const float* __restrict__ bias, float* __restrict__ out, int K, int Nn) {
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
  const int pr = perm ? perm[row] : row;        // -1: a padding row (reads as zeros)
  const int kk = pr >= 0 ? K : 0;
  const float* a = A + (size_t)(pr >= 0 ? (perm ? pr / gk : pr) : 0) * K;
  const float* w = W + (size_t)seg * Nn * K + (size_t)col * K;
  float acc = 0.f;
  for (int j = 0; j < kk; ++j) acc = fmaf(a[j], w[j], acc);
  float v;
  if (MODE == MODE_SWIGLU_UP) {
    const float* w3 = W3 + (size_t)seg * Nn * K + (size_t)col * K;
    float acc3 = 0.f;
    for (int j = 0; j < kk; ++j) acc3 = fmaf(a[j], w3[j], acc3);
    v = silu_f(acc) * acc3;
  } else {
    v = acc;
    if (HAS_BIAS) v += bias[(size_t)seg * Nn + col];
    if (MODE == MODE_GELU_UP) v = gelu_f(v);
  }
  out[i] = v;
}

hipError_t launch_build_tiles(const int32_t* offsets, int n_seg, int dense_rows, int32_t* big, int max_big,
                              int32_t* small, int max_small, int kind, hipStream_t s) {
  if (n_seg > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, n_seg, dense_rows, big, max_big, small,
                     max_small, kind);
  return hipGetLastError();
}

int grouped_gemm_max_tiles(int max_rows, int n_seg) { return max_rows / 256 + n_seg; }
int grouped_gemm_max_small_tiles(int max_rows, int n_seg) { return max_rows / 64 + n_seg; }
size_t grouped_gemm_partials_bytes() {
  return (size_t)kMaxSplitUnits * (kBM2P + kBM3) * kBN2 * sizeof(float);
}
size_t grouped_gemm_gather_max_bytes() { return (size_t)kOobOffset - (1u << 20); }

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

template <int MODE, bool HAS_BIAS, bool GATHER, bool FP8 = false>
static void launch_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const int cols = MODE == MODE_SWIGLU_UP ? kBN2 / 2 : kBN2;
  GemmParams p;
  p.A = (const uint16_t*)g.a;
  p.perm = g.perm;
  p.gk = g.gather_k > 0 ? g.gather_k : 1;
  p.a_bytes = GATHER ? (uint32_t)((size_t)g.a_rows * g.K * 2) : 0u;
  p.offsets = g.offsets;
  p.n_seg = g.n_seg;
  p.dense_rows = g.max_rows;
  // routed segments: the 256-row / 64-row split of each expert's tail is chosen on the device
  p.kind = FP8 ? 1 : (g.offsets == nullptr || MODE == MODE_LOGITS ? 0 : (MODE == MODE_DOWN ? 4 : 3));
  // short tails ride on whole 256-row tiles (the attached-row epilogue covers these modes)
  p.attach = !FP8 && (MODE == MODE_SWIGLU_UP || MODE == MODE_GELU_UP || (MODE == MODE_DOWN && g.comb_out == nullptr));
  p.W = (const uint16_t*)g.w;
  p.W3 = (const uint16_t*)g.w3;
  p.bias = (const uint16_t*)g.bias;
  p.out = (uint16_t*)g.out;
  p.pre = (MODE == MODE_SWIGLU_UP || MODE == MODE_GELU_UP) ? (uint16_t*)g.pre : nullptr;
  p.pre_plane = (long long)g.max_rows * g.Nn;
  p.cmb.perm = g.comb_perm;
  p.cmb.gates = g.comb_gates;
  p.cmb.residual = (const uint16_t*)g.comb_residual;
  p.cmb.shared_y = (const uint16_t*)g.comb_shared;
  p.cmb.out = MODE == MODE_DOWN ? (uint16_t*)g.comb_out : nullptr;
  p.out_f = g.out_f32;
  p.bias_f = g.bias_f32;
  p.W8 = g.w8;
  p.W8_3 = g.w8_3;
  p.scale1 = g.scale1;
  p.scale3 = g.scale3;
  p.partials = g.partials;
  p.partials_small = g.partials + (size_t)kMaxSplitUnits * kBM2P * kBN2;
  p.K = g.K;
  p.Nn = g.Nn;
  p.n_ntiles = (g.Nn + cols - 1) / cols;
  const int grid = ((device_cus() + kXcds - 1) / kXcds) * kXcds;
  // fp8 weights use 64-row tiles only; with fewer than kBigTailMin rows no segment has a 256-row tile
  bool run_big = !FP8 && g.max_rows >= kBigTailMin, run_small = true, run_fixup = true;
  if (g.offsets == nullptr) {   // one dense segment of max_rows rows: the host knows both tile counts and plans
    int nb = 0, ns = 0;
    seg_tiles(g.max_rows, p.attach && p.kind == 0 ? 5 : p.kind, nb, ns);
    const int KT = g.K / kBK2;
    run_big = nb > 0;
    run_small = ns > 0;
    run_fixup = plan_units(nb * p.n_ntiles, grid, KT).rem > 0 || plan_units(ns * p.n_ntiles, grid, KT).rem > 0;
  }
  if (run_big)
    hipLaunchKernelGGL((grouped_gemm_big_kernel<MODE, HAS_BIAS, GATHER>), dim3(grid), dim3(512), 0, s, p);
  if (run_small)
    hipLaunchKernelGGL((grouped_gemm_small_kernel<MODE, HAS_BIAS, GATHER, FP8>), dim3(grid), dim3(256), 0, s, p);
  if (run_fixup && !(MODE == MODE_LOGITS && g.no_fixup))
    hipLaunchKernelGGL((split_fixup_kernel<MODE, HAS_BIAS>), dim3(2 * grid), dim3(256), 0, s, p, grid);
}

template <int MODE, bool HAS_BIAS>
static void launch_f32(const GroupedGemmArgs& g, hipStream_t s) {
  const size_t n = (size_t)g.max_rows * g.Nn;
  hipLaunchKernelGGL((grouped_gemm_f32_kernel<MODE, HAS_BIAS>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                     0, s, (const float*)g.a, g.perm, g.gather_k > 0 ? g.gather_k : 1, g.offsets, g.n_seg,
                     g.max_rows, (const float*)g.w, (const float*)g.w3, (const float*)g.bias, (float*)g.out, g.K,
                     g.Nn);
}

LogitParts logits_parts(const GroupedGemmArgs& g) {
  // the plans launch_bf16 gives the two kernels for one dense segment (tile kind 0)
  LogitParts z{};
  const int grid = ((device_cus() + kXcds - 1) / kXcds) * kXcds;
  const int KT = g.K / kBK2, n_ntiles = (g.Nn + kBN2 - 1) / kBN2;
  seg_tiles(g.max_rows, 0, z.nb, z.ns);
  const UnitPlan pb = plan_units(z.nb * n_ntiles, grid, KT), ps = plan_units(z.ns * n_ntiles, grid, KT);
  z.logits = g.out_f32;
  z.part_big = g.partials;
  z.part_small = g.partials + (size_t)kMaxSplitUnits * kBM2P * kBN2;
  z.rows_big = kBM2P;
  z.bias = g.bias_f32;
  z.full_b = pb.full;
  z.s_b = pb.s;
  z.full_s = ps.full;
  z.s_s = ps.s;
  z.ld = kBN2;
  return z;
}

hipError_t launch_grouped_gemm(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.max_rows <= 0) return hipSuccess;
  if (g.comb_out && (g.dtype != MOE_BF16 || g.mode != MODE_DOWN || !g.comb_perm || !g.comb_gates))
    return hipErrorInvalidValue;
  const bool hb = g.bias != nullptr;
  if (g.dtype == MOE_F32) {
    if (g.mode == MODE_SWIGLU_UP) launch_f32<MODE_SWIGLU_UP, false>(g, s);
    else if (g.mode == MODE_GELU_UP) hb ? launch_f32<MODE_GELU_UP, true>(g, s) : launch_f32<MODE_GELU_UP, false>(g, s);
    else hb ? launch_f32<MODE_DOWN, true>(g, s) : launch_f32<MODE_DOWN, false>(g, s);
    return hipGetLastError();
  }
  const bool gather = g.perm != nullptr;
  if (gather && (g.mode == MODE_LOGITS || (size_t)g.a_rows * g.K * 2 > grouped_gemm_gather_max_bytes()))
    return hipErrorInvalidValue;
  if (g.mode == MODE_LOGITS && (g.Nn % 8 != 0 || g.n_seg != 1)) return hipErrorInvalidValue;
  if (g.no_fixup && (g.mode != MODE_LOGITS || g.offsets != nullptr || g.Nn > kBN2)) return hipErrorInvalidValue;
  if (g.fp8 && (g.mode == MODE_LOGITS || (g.mode != MODE_DOWN && !gather) || !g.w8 || !g.scale1 ||
                (g.mode == MODE_SWIGLU_UP && (!g.w8_3 || !g.scale3))))
    return hipErrorInvalidValue;
  if (g.n_seg < 1 || g.n_seg > kMaxExperts) return hipErrorInvalidValue;
  if (g.fp8) {   // fp8 weights: up with the row gather, or down
    if (g.mode == MODE_SWIGLU_UP) launch_bf16<MODE_SWIGLU_UP, false, true, true>(g, s);
    else if (g.mode == MODE_GELU_UP)
      hb ? launch_bf16<MODE_GELU_UP, true, true, true>(g, s) : launch_bf16<MODE_GELU_UP, false, true, true>(g, s);
    else hb ? launch_bf16<MODE_DOWN, true, false, true>(g, s) : launch_bf16<MODE_DOWN, false, false, true>(g, s);
    return hipGetLastError();
  }
  if (g.mode == MODE_SWIGLU_UP) {
    gather ? launch_bf16<MODE_SWIGLU_UP, false, true>(g, s) : launch_bf16<MODE_SWIGLU_UP, false, false>(g, s);
  } else if (g.mode == MODE_GELU_UP) {
    if (hb) gather ? launch_bf16<MODE_GELU_UP, true, true>(g, s) : launch_bf16<MODE_GELU_UP, true, false>(g, s);
    else gather ? launch_bf16<MODE_GELU_UP, false, true>(g, s) : launch_bf16<MODE_GELU_UP, false, false>(g, s);
  } else if (g.mode == MODE_DOWN) {
    if (gather)   // plain product of gathered token rows (the backward recomputes pre-activations)
      hb ? launch_bf16<MODE_DOWN, true, true>(g, s) : launch_bf16<MODE_DOWN, false, true>(g, s);
    else hb ? launch_bf16<MODE_DOWN, true, false>(g, s) : launch_bf16<MODE_DOWN, false, false>(g, s);
  } else {
    g.bias_f32 ? launch_bf16<MODE_LOGITS, true, false>(g, s) : launch_bf16<MODE_LOGITS, false, false>(g, s);
  }
  return hipGetLastError();
}

}  // namespace moe
