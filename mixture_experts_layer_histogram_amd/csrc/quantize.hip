// fp8 (OCP E4M3) weight-only quantisation of expert weights.
//
// [S] "How sparse models scale": the memory of large MoE models is the
// obstacle, and 8-bit (or 4-bit) weights are how they are run on fewer
// devices.  Here each output row of a weight matrix stored [out, in] gets one
// fp32 scale: amax = max |w|, scale = amax / 448, and every element becomes
// the E4M3 code nearest to w * (448 / amax) (ties to the even code,
// magnitudes above 448 saturate).  All arithmetic is fp32 with correctly
// rounded division, so the codes are a deterministic function of the weights.
#include "moe_internal.h"

#include <math.h>

namespace moe {

// E4M3 code nearest to x (|x| <= 448 expected; larger magnitudes saturate).
// Subnormals are multiples of 2^-9 below 2^-6; normals have 3 mantissa bits.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);   // 0..8; 8 is the code of 2^-6
  const uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFFu) - 127;                          // -6 .. 8
  const float mant = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u);
  int m = (int)rintf((mant - 1.0f) * 8.0f);                         // 0 .. 8
  if (m == 8) { m = 0; e += 1; }
  return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)m;
}

// One wavefront per row: the row maximum by a wave reduction (max is exact in
// any order), then each lane quantises its elements, four codes per store.
__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const uint16_t* __restrict__ w, long long rows,
                                                                int cols, uint8_t* __restrict__ q,
                                                                float* __restrict__ scales) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint16_t* src = w + (size_t)row * cols;
  float amax = 0.f;
  for (int c = lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(bf16_to_f32(src[c])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  uint8_t* dst = q + (size_t)row * cols;
  if (cols % 4 == 0) {
    for (int c = lane * 4; c < cols; c += 64 * 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(src + c);
      const uint32_t c0 = e4m3_rne(bf16_to_f32((uint16_t)(v.x & 0xFFFFu)) * inv);
      const uint32_t c1 = e4m3_rne(bf16_to_f32((uint16_t)(v.x >> 16)) * inv);
      const uint32_t c2 = e4m3_rne(bf16_to_f32((uint16_t)(v.y & 0xFFFFu)) * inv);
      const uint32_t c3 = e4m3_rne(bf16_to_f32((uint16_t)(v.y >> 16)) * inv);
      *reinterpret_cast<uint32_t*>(dst + c) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  } else {
    for (int c = lane; c < cols; c += 64) dst[c] = (uint8_t)e4m3_rne(bf16_to_f32(src[c]) * inv);
  }
  if (lane == 0) scales[row] = scale;
}

hipError_t launch_quantize_fp8(const uint16_t* w, long long rows, int cols, uint8_t* q, float* scales,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, w, rows, cols,
                     q, scales);
  return hipGetLastError();
}

}  // namespace moe
