// fa_tile.hpp — an LDS tile of 16-bit rows (head dimension D) that is read both by rows (an MFMA
// operand with the head dimension as k) and transposed (an operand with the rows as k, in the
// order a 32x32 accumulator holds its rows).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

// The tile layout (row-major, 16-byte chunks XOR-ed by swz of the row) and the per-lane offsets
// of its row reads and transpose reads.
template <int D>
struct OpTile {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = 64 * ROWB;     // 64 rows
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  // Chunk swizzle, free of bank conflicts (64 banks of 4 bytes) for both kinds of read:
  //  * a row read serves 16 lanes = 16 consecutive rows at one logical chunk per cycle; rows that
  //    start on the same bank (every second row for 128-byte rows, every row for 256-byte rows)
  //    must see distinct values of swz;
  //  * a transpose read serves 32 lanes = 4 consecutive rows (4-aligned) x one aligned group of 4
  //    chunks; rows that start on the same bank must differ in bit 2 (and 3) of swz, which moves
  //    them to another group of 4 chunks.
  // swz is unchanged by adding 16 rows and changed by adding 8.
  __device__ static int swz(int r) {
    return ROWB == 128 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
  }
  // Row read (A or B operand with the head dimension as k): row r (0..31 of a 32-row block),
  // k-slots ks*16 + hl*8 .. +7.
  __device__ static int row_off(int r, int ks, int hl) { return r * ROWB + (((2 * ks + hl) ^ swz(r)) << 4); }
  // Transpose read (A operand with the rows as k): for 16-lane group g16 and lane s16 = 4 tr + tc,
  // rows 4 (g16 >> 1) + tr (+ 8 e8), columns db*32 + (g16 & 1)*16 + 4 tc .. +3. Adding 16 or 32
  // rows keeps the swizzle, adding 8 changes it, so each column block has two offsets.
  __device__ static int tr_off(int lane, int db, int e8) {
    const int g16 = lane >> 4, s16 = lane & 15, tr = s16 >> 2, tc = s16 & 3;
    const int row = 4 * (g16 >> 1) + tr;
    const int chunk = db * 4 + (g16 & 1) * 2 + (tc >> 1);
    return row * ROWB + ((chunk ^ swz(row + 8 * e8)) << 4) + (tc & 1) * 8;
  }
};

// A operand of a product whose k runs over 16 tile rows (block of 32 rows kb, half 'half'):
// rows kb*32 + half*16 + (t / 4) * 8 + (l / 32) * 4 + t % 4 for k-slot (l / 32) * 8 + t, i.e. the
// order in which a 32x32 accumulator holds its rows, so that an accumulator packed to 16 bits is
// the matching B operand.
// `base` holds the slot's address plus the lane's two offsets (tr_bases), so that the block and
// half land in the reads' immediate offsets.
template <int D>
__device__ inline i32x4 tr_operand(const uint32_t (&base)[D / 32][2], int kb, int half, int db) {
  constexpr int ROWB = D * 2;
  const i32x2 v0 = lds_read_tr16(base[db][0] + (kb * 32 + half * 16) * ROWB);
  const i32x2 v1 = lds_read_tr16(base[db][1] + (kb * 32 + half * 16 + 8) * ROWB);
  return i32x4{v0[0], v0[1], v1[0], v1[1]};
}

template <int D>
__device__ inline void tr_bases(uint32_t slot, const int (&toff)[D / 32][2], uint32_t (&base)[D / 32][2]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e8 = 0; e8 < 2; ++e8) base[db][e8] = opaque_vbase(slot + toff[db][e8]);
}

}  // namespace fa
