// fa_device.hpp — device-side helpers shared by the forward kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// f(Int<0>{}), ..., f(Int<N-1>{}): a loop whose index is a compile-time constant in every trip
// (for long bodies the unroller may otherwise keep a loop, and arrays indexed by its counter
// then live in scratch memory).
template <int I>
struct Int {
  static constexpr int value = I;
};
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr float kLn2 = 0.69314718055994530942f;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Block index -> logical block index, so that each XCD's share is one contiguous range.
__device__ inline int xcd_remap(int id, int n) {
  const int xcd = id & 7, k = id >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// Which (batch, head, tile) workgroup `id` of a launch of n = (batch x heads) x num_tiles
// computes. Heads are enumerated batch-major (inside a batch the query heads sharing a K/V head
// are consecutive); under a causal mask tile t is the longest of its head when t = num_tiles - 1
// and the shortest when t = 0. Blocks are dealt round-robin over the 8 XCDs.
//  * No causal mask: head by head, each XCD one contiguous range of heads (xcd_remap), so a
//    head's K/V stays in one XCD's L2.
//  * Causal, heads a multiple of 8: each XCD takes a contiguous range of whole heads and goes
//    through them by chunks of up to kChunk heads (a divisor of its head count; one K/V head
//    under 4-way GQA), longest tiles of the chunk first: the chunk in flight keeps the XCD's L2
//    working set small, every XCD gets the same mix of long and short tiles, and the longest
//    work starts first, which keeps the launch's tail short.
//  * Causal otherwise, and packed batches of sequences of different lengths (`spread`: whole
//    sequences on one XCD would leave the XCDs unequally loaded): highest tiles of every head
//    first, consecutive ids on different XCDs.
__device__ inline void schedule_block(int id, int n, int num_tiles, int H, bool causal, int* b, int* h, int* t,
                                      bool spread = false) {
  constexpr int kChunk = 4;
  const int n_bh = n / num_tiles;
  int bh;
  if (spread) {
    const int rank = id / n_bh;
    bh = id - rank * n_bh;
    *t = num_tiles - 1 - rank;
  } else if (!causal) {
    const int L = xcd_remap(id, n);
    bh = L / num_tiles;
    *t = L - bh * num_tiles;
  } else if (n_bh % 8 == 0) {
    const int hx = n_bh / 8;   // heads per XCD
    const int c = hx % kChunk == 0 ? kChunk : (hx % 2 == 0 ? 2 : 1);
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

// Value of x held by lane l ^ 32, combined with x: max or sum over the lane pair.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte-per-lane HBM -> LDS load (buffer_load_dwordx4 ... lds): lane l's 16 bytes land at
// LDS byte address lds_addr + 16 * l. Written out here rather than through the compiler's
// builtin because the compiler's wait-count pass, unable to tell LDS ring slots apart, would put a
// blanket vmcnt(0) in front of the V transpose reads and undo the prefetch. The kernel waits for
// these loads itself (vmcnt before each barrier). There is no destination register: nothing in the
// register file is left pending. M0 (which addresses the LDS side) is saved and restored inside
// the block, so the compiler's view of it never changes; the s_nop is the wait state between a
// write of M0 and its use by the load. The LDS address and the offset are wave-uniform; they pass
// through readfirstlane because the compiler sometimes keeps a uniform loop value in a vector
// register, and the instruction takes scalar operands only.
struct BufDesc {
  uint32_t w[4];
};
__device__ inline BufDesc make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return BufDesc{{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, kRsrcWord3}};
}
__device__ inline void dma16(const BufDesc& d, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 rs = u32x4{d.w[0], d.w[1], d.w[2], d.w[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}
// The 4-byte form: lane l's 4 bytes land at LDS byte address lds_addr + 4 * l.
__device__ inline void dma4(const BufDesc& d, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 rs = u32x4{d.w[0], d.w[1], d.w[2], d.w[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}
// LDS reads addressed by 32-bit LDS byte addresses. Going through an integer address (instead of a
// generic pointer) lets the compiler put constant displacements into the instruction's offset field
// instead of recomputing each address with vector adds.
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ inline i32x4 lds_read_b128(uint32_t addr) { return *(const lds_i32x4*)(uintptr_t)addr; }
__device__ inline i32x2 lds_read_tr16(uint32_t addr) {
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr));
}
__device__ inline i32x2 lds_read_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)addr);
}
// Hides a per-lane LDS base address from the optimiser. Without it, the compiler reassociates
// base + lane_offset + constant into base + (lane_offset + constant) with one register per
// constant, and every read pays a vector add; with an opaque base the constant stays in the
// instruction's offset field.
__device__ inline uint32_t opaque_vbase(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ inline uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace fa
