// fa_f16_common.hpp — pieces shared by the fp16 / bf16 forward kernels: MFMA and packing traits
// of the two storage types, the softmax reference bound, and the LDS swizzles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

struct F16 {
  static constexpr int kDtype = 0;
  __device__ static inline f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  __device__ static inline uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
  }
  // Row-sum contribution of a pair: the fp32 values, the pair's sum first. (Summing the
  // fp16-rounded pair with one v_dot2c_f32_f16 against (1, 1) is half the instructions, but its
  // chain of dependent accumulations measured 0.6-2% slower than these adds.)
  __device__ static inline float sum2(float acc, uint32_t, float x, float y) { return acc + (x + y); }
};

struct BF16 {
  static constexpr int kDtype = 1;
  __device__ static inline f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
  }
  // bf16 rounding of p is too coarse for a 1e-3 lse: the row sum uses the fp32 values.
  __device__ static inline float sum2(float acc, uint32_t, float x, float y) { return acc + (x + y); }
};

// Softmax reference. p = exp2(s * c - m) is computed against the row's current reference m
// without first taking the tile's row max. If every p of the tile is at most 2^15 (checked
// through the row sum, which bounds each term), the tile is done: the products and sums use the
// same m as the final division and the lse, so the result is unchanged, and p stays inside the
// fp16 range. Otherwise (the first tile of a row, where m = -inf, or a score far above every
// earlier one) the wave takes the slow path: m moves to the running max, O and l are rescaled
// by exp2(m_old - m_new), and p is recomputed.
constexpr float kSumBound = 32768.f;

// LDS bank model of gfx950: 64 banks of 4 bytes, a 128-bit read served 16 lanes (256 bytes) per
// cycle. Swizzles below are XORs on the 16-byte chunk index of a row; they make
//  * the K reads (16 consecutive rows, one chunk each) hit 16 distinct 16-byte bank groups,
//  * the V transpose reads (4 rows x 64 bytes per 32 lanes) hit distinct bank groups,
//  * the row-major tile writes stay conflict-free (a row's chunks are only permuted).
template <int ROWB>
__device__ inline int k_swz(int row) {
  return ROWB == 128 ? (row >> 1) & 7 : row & 15;
}
template <int ROWB>
__device__ inline int v_swz(int row) {
  return ROWB == 128 ? (row & 3) << 1 : (row & 3) << 2;
}

}  // namespace fa
