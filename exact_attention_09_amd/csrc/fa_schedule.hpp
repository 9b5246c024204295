// fa_schedule.hpp — which (batch, head, tile) each workgroup of a launch computes. Host and
// device: the kernels call it, and the C ABI exports it (fa_block_order) so that the order can be
// checked on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Unsigned division by a launch constant d >= 1 for dividends below 2^31, with host-computed
// constants: q = (umulhi(n, m) + n) >> s, s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1
// (the round-up method of Granlund and Montgomery; exact on that range, checked on the host).
// On the device it is three scalar instructions where a generic 32-bit division takes about 30
// with a float reciprocal on the vector unit.
struct FastDiv {
  uint32_t d, m, s;
};
__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while (s < 31 && (1u << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}
__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (t + n) >> f.s;
}

// Block index -> logical block index, so that each XCD's share is one contiguous range.
__host__ __device__ inline int xcd_remap(int id, int n) {
  const int xcd = id & 7, k = id >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// Which (batch, head, tile) each workgroup of a launch of n = (batch x heads) x num_tiles
// computes. Heads are enumerated batch-major (inside a batch the `group` query heads sharing a
// K/V head are consecutive); under a causal mask tile t is the longest of its head when
// t = num_tiles - 1 and the shortest when t = 0. Blocks are dealt round-robin over the 8 XCDs
// (block id -> XCD id % 8), and a head's K/V is read from the L2 of the XCD that runs it.
//  * No causal mask: head by head, each XCD one contiguous range of heads (xcd_remap), so a
//    head's K/V stays in one XCD's L2.
//  * Causal, heads a multiple of 8: each XCD takes a contiguous range of whole heads and goes
//    through them by chunks of up to 4 heads (a divisor of its head count; one K/V head under
//    4-way GQA), longest tiles of the chunk first: the chunk in flight keeps the XCD's L2
//    working set small, every XCD gets the same mix of long and short tiles, and the longest
//    work starts first, which keeps the launch's tail short.
//  * Packed batches of sequences of different lengths (`packed`), K/V heads per sequence a
//    multiple of 8: the K/V heads u = (batch, K/V head) are dealt to the XCDs in turn (u to XCD
//    u % 8), so every XCD gets the same share of every sequence, and each XCD goes through its
//    query heads by chunks as above, highest tiles first: the chunk in flight is a few heads of
//    one sequence, whose K/V fits the XCD's L2.
//  * Otherwise: highest tiles of every head first, consecutive ids on different XCDs.
// The mode and the divisions by launch constants are fixed on the host (make_schedule), so the
// kernels' start-up is a few scalar multiplies.
struct Schedule {
  int mode;                 // kSchedInterleaved, kSchedRanked, kSchedHeads, kSchedChunked
  int n, num_tiles, lc;     // lc = log2 of the chunk's head count
  FastDiv tiles, bh, per, heads, group;   // num_tiles, heads * batches, chunk * num_tiles, H, group
};
constexpr int kSchedInterleaved = 0, kSchedRanked = 1, kSchedHeads = 2, kSchedChunked = 3;

inline Schedule make_schedule(int n, int num_tiles, int H, int group, bool causal, bool packed) {
  Schedule S;
  S.n = n;
  S.num_tiles = num_tiles;
  const int n_bh = n / num_tiles;
  const int hx = n_bh / 8;   // heads per XCD
  const int c = hx % 4 == 0 ? 4 : (hx % 2 == 0 ? 2 : 1);
  if (packed && (H / group) % 8 == 0) S.mode = kSchedInterleaved;
  else if (packed) S.mode = kSchedRanked;
  else if (!causal) S.mode = kSchedHeads;
  else if (n_bh % 8 == 0) S.mode = kSchedChunked;
  else S.mode = kSchedRanked;
  S.lc = c == 4 ? 2 : (c == 2 ? 1 : 0);
  S.tiles = make_fastdiv((uint32_t)num_tiles);
  S.bh = make_fastdiv((uint32_t)n_bh);
  S.per = make_fastdiv((uint32_t)(c * num_tiles));
  S.heads = make_fastdiv((uint32_t)H);
  S.group = make_fastdiv((uint32_t)group);
  return S;
}

__host__ __device__ inline void schedule_block(int id, const Schedule& S, int* b, int* h, int* t) {
  uint32_t bh, rank;
  if (S.mode == kSchedHeads) {
    const uint32_t L = (uint32_t)xcd_remap(id, S.n);
    bh = fdiv(L, S.tiles);
    *t = (int)(L - bh * (uint32_t)S.num_tiles);
  } else if (S.mode == kSchedRanked) {
    rank = fdiv((uint32_t)id, S.bh);
    bh = (uint32_t)id - rank * S.bh.d;
    *t = S.num_tiles - 1 - (int)rank;
  } else {
    // kSchedChunked: the XCD's share in order (xcd_remap); kSchedInterleaved: the k-th block the
    // XCD id % 8 receives
    const uint32_t L = S.mode == kSchedChunked ? (uint32_t)xcd_remap(id, S.n) : (uint32_t)id >> 3;
    const uint32_t chunk = fdiv(L, S.per), r = L - chunk * S.per.d;
    rank = r >> S.lc;
    const uint32_t pi = (chunk << S.lc) + (r & ((1u << S.lc) - 1));   // head number within the share
    if (S.mode == kSchedChunked) {
      bh = pi;
    } else {   // query head pi of the XCD's list: K/V head pi / group of the XCD, dealt every 8th
      const uint32_t u = fdiv(pi, S.group);
      bh = ((u << 3) + ((uint32_t)id & 7)) * S.group.d + (pi - u * S.group.d);
    }
    *t = S.num_tiles - 1 - (int)rank;
  }
  const uint32_t bb = fdiv(bh, S.heads);
  *b = (int)bb;
  *h = (int)(bh - bb * S.heads.d);
}

}  // namespace fa
