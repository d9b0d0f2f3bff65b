// Device helpers of the gfx950 quantized-attention kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_launch.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 values from one 16-byte word.
__device__ __forceinline__ void unpack8(const uint4& u, float f[8]) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// Correctly rounded x / s from r = RN(1 / s): q0 = RN(x r) is within an ulp
// of x / s and the residual q0 s - x is exact in an fma, so one correction
// step gives RN(x / s) (Markstein's theorem). The residual is formed as
// q0 s - x so that x = -0 keeps its sign, as in a division. With
// s >= 2^-60 the residual cannot underflow unless |x / s| < 2^-24, where
// int8 and E4M3 codes are 0 whichever way the quotient rounds; below that
// scale the caller divides.
constexpr float kFastDivMinScale = 0x1p-60f;
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
}

// INT8 block code of a quotient already rounded to fp32: round half to even,
// clamp to [-127, 127].
__device__ __forceinline__ uint32_t code_i8(float q) {
  return (uint32_t)(int)fminf(fmaxf(rintf(q), -127.0f), 127.0f) & 0xFFu;
}

// Byte offset of 16-byte chunk `chunk` of key row `key` in an LDS K tile of
// 64 rows x D bytes. The XOR swizzle is linear in the key bits and was chosen
// so that the A-operand reads of the QK step (16 bytes per lane) and the
// staging writes touch distinct 16-byte bank groups both per 8 lanes in a
// 128-byte window and per 16 lanes in a 256-byte window.
template <int D>
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
  int swz;
  if (D == 128)
    swz = ((key >> 1) & 1) | (((key ^ (key >> 2)) & 1) << 1) | (((key >> 5) & 1) << 2);
  else
    swz = (((key >> 1) ^ (key >> 2)) & 1) | (((key >> 5) & 1) << 1);
  return key * D + ((chunk ^ swz) << 4);
}

// Byte offset of 16-byte chunk `chunk` (0..3) of channel row `c` in an LDS V
// tile of D rows x 64 key bytes (same two bank-group conditions).
__device__ __forceinline__ int v_lds_off(int c, int chunk) {
  return c * 64 + ((chunk ^ (((c >> 1) ^ (c >> 2)) & 3)) << 4);
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a wave's LDS staging
// area for its 32 bf16 output rows (2D bytes each). The chunk index is XORed
// with row bits so that the register-layout writes (one 8-byte half chunk per
// lane, 32 rows at once) fall in at most two lanes per bank and the row-order
// reads (16 lanes per 256 bytes) in one.
template <int D>
__device__ __forceinline__ int out_lds_off(int row, int chunk) {
  const int f = D == 128 ? (row & 15) : ((row >> 1) & 7);
  return row * 2 * D + ((chunk ^ f) << 4);
}

// A-operand row -> key mapping of the QK matrix-core step. The 32x32 int32
// result gives lane (h = lane/32, q = lane%32), register r the row
// 8*(r/4) + 4*h + (r%4). Loading key 32*h + 16*m + 4*(row/8) + (row%4) for
// row = 8*(row/8) + 4*h + (row%4) makes register r of half h hold key
// 32*h + 16*m + r: each lane ends with 32 consecutive keys of one query.
__device__ __forceinline__ int qk_row_key(int row, int m) {
  return 32 * ((row >> 2) & 1) + 16 * m + 4 * (row >> 3) + (row & 3);
}

}  // namespace sage
