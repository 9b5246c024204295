// fa_schedule.hpp — which (batch, head, tile) each workgroup of a launch computes. Host and
// device: the kernels call it, and the C ABI exports it (fa_block_order) so that the order can be
// checked on the host.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// Block index -> logical block index, so that each XCD's share is one contiguous range.
__host__ __device__ inline int xcd_remap(int id, int n) {
  const int xcd = id & 7, k = id >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// Which (batch, head, tile) workgroup `id` of a launch of n = (batch x heads) x num_tiles
// computes. Heads are enumerated batch-major (inside a batch the `group` query heads sharing a
// K/V head are consecutive); under a causal mask tile t is the longest of its head when
// t = num_tiles - 1 and the shortest when t = 0. Blocks are dealt round-robin over the 8 XCDs
// (block id -> XCD id % 8), and a head's K/V is read from the L2 of the XCD that runs it.
//  * No causal mask: head by head, each XCD one contiguous range of heads (xcd_remap), so a
//    head's K/V stays in one XCD's L2.
//  * Causal, heads a multiple of 8: each XCD takes a contiguous range of whole heads and goes
//    through them by chunks of up to kChunk heads (a divisor of its head count; one K/V head
//    under 4-way GQA), longest tiles of the chunk first: the chunk in flight keeps the XCD's L2
//    working set small, every XCD gets the same mix of long and short tiles, and the longest
//    work starts first, which keeps the launch's tail short.
//  * Packed batches of sequences of different lengths (`packed`), K/V heads per sequence a
//    multiple of 8: the K/V heads u = (batch, K/V head) are dealt to the XCDs in turn (u to XCD
//    u % 8), so every XCD gets the same share of every sequence, and each XCD goes through its
//    query heads by chunks as above, highest tiles first: the chunk in flight is a few heads of
//    one sequence, whose K/V fits the XCD's L2.
//  * Otherwise: highest tiles of every head first, consecutive ids on different XCDs.
__host__ __device__ inline void schedule_block(int id, int n, int num_tiles, int H, int group, bool causal,
                                               bool packed, int* b, int* h, int* t) {
  constexpr int kChunk = 4;
  const int n_bh = n / num_tiles;
  auto chunk_of = [](int hx) { return hx % kChunk == 0 ? kChunk : (hx % 2 == 0 ? 2 : 1); };
  int bh;
  if (packed && (H / group) % 8 == 0) {
    const int x = id & 7, k = id >> 3;
    const int hx = n_bh / 8;   // query heads per XCD: n_bh / (8 group) K/V heads of `group` each
    const int c = chunk_of(hx);
    const int per = c * num_tiles;
    const int chunk = k / per, r = k - chunk * per;
    const int rank = r / c;
    const int pi = chunk * c + (r - rank * c);   // the XCD's query head pi: K/V head pi / group of the XCD
    bh = ((pi / group) * 8 + x) * group + pi % group;
    *t = num_tiles - 1 - rank;
  } else if (packed) {
    const int rank = id / n_bh;
    bh = id - rank * n_bh;
    *t = num_tiles - 1 - rank;
  } else if (!causal) {
    const int L = xcd_remap(id, n);
    bh = L / num_tiles;
    *t = L - bh * num_tiles;
  } else if (n_bh % 8 == 0) {
    const int hx = n_bh / 8;   // heads per XCD
    const int c = chunk_of(hx);
    const int L = xcd_remap(id, n);
    const int per = c * num_tiles;
    const int chunk = L / per, r = L - chunk * per;
    const int rank = r / c;
    bh = chunk * c + (r - rank * c);
    *t = num_tiles - 1 - rank;
  } else {
    const int rank = id / n_bh;
    bh = id - rank * n_bh;
    *t = num_tiles - 1 - rank;
  }
  *b = bh / H;
  *h = bh - *b * H;
}

}  // namespace fa
