// fa_mask.hpp — which keys a query row may attend to, and how K/V tiles are classified.
//
// Causal masking and the (left, right) sliding window of the pages' interface ("Flash Attention -
// Fast Memory-Efficient Attention", skill page, Workflow 2 Steps 2-3). With off = Nk - Nq, query
// row i admits key j iff
//     lo(i) <= j <= hi(i),
//     lo(i) = wl < 0 ? 0 : max(0, i + off - wl),
//     hi(i) = min(Nk - 1, i + off + right),  right = causal ? 0 : wr  (wr < 0: unbounded).
// Causal with a right window is their intersection, whose right reach is min(wr, 0) = 0.
// Both bounds are non-decreasing in i, so for a block of rows [r0, r1]:
//   * a tile [j0, j1] is admitted for every pair iff lo(r1) <= j0 and j1 <= hi(r0);
//   * it holds no admitted pair if j1 < lo(r0) or j0 > hi(r1);
//   * otherwise it is partial and the kernel masks it element by element.
// The same functions plan the launch on the host and steer the kernel's tile loop.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fa {

struct MaskSpec {
  int Nq, Nk, causal, wl, wr;
};

__host__ __device__ inline int64_t key_lo(const MaskSpec& m, int64_t i) {
  if (m.wl < 0) return 0;
  int64_t v = i + (int64_t)(m.Nk - m.Nq) - m.wl;
  return v < 0 ? 0 : v;
}

__host__ __device__ inline int64_t key_hi(const MaskSpec& m, int64_t i) {
  int64_t right = m.causal ? 0 : m.wr;
  if (right < 0) return m.Nk - 1;
  int64_t v = i + (int64_t)(m.Nk - m.Nq) + right;
  return v > m.Nk - 1 ? m.Nk - 1 : v;
}

enum TileClass { TILE_SKIP = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

// Rows [r0, r1] (inclusive, r1 < Nq) against keys [j0, j0 + bn - 1].
__host__ __device__ inline int classify_tile(const MaskSpec& m, int r0, int r1, int j0, int bn) {
  int64_t j1 = (int64_t)j0 + bn - 1;
  if (j1 < key_lo(m, r0) || j0 > key_hi(m, r1)) return TILE_SKIP;
  if (key_lo(m, r1) <= j0 && j1 <= key_hi(m, r0)) return TILE_FULL;
  return TILE_PARTIAL;
}

// K/V tiles [*tb, *te) that can hold an admitted key for rows [r0, r1].
__host__ __device__ inline void tile_range(const MaskSpec& m, int r0, int r1, int bn, int* tb, int* te) {
  int64_t lo = key_lo(m, r0), hi = key_hi(m, r1);
  if (hi < lo || hi < 0 || lo > m.Nk - 1) {
    *tb = *te = 0;
    return;
  }
  *tb = (int)(lo / bn);
  *te = (int)(hi / bn) + 1;
}

}  // namespace fa
