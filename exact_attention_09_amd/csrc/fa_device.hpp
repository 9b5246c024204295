// fa_device.hpp — device-side helpers shared by the forward kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_schedule.hpp"

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
// write of M0 and its use by the load. The LDS address is wave-uniform; it passes through
// readfirstlane because the compiler sometimes keeps a uniform loop value in a vector register,
// and the instruction takes scalar operands only.
//
// Bounds. On this family the buffer range check compares only the per-lane (VGPR) offset with
// the descriptor's byte count; an offset given in the instruction's scalar field is added after
// the check. A tile's byte offset (`soff`, wave-uniform) therefore moves the descriptor itself:
// its base advances by soff and its byte count shrinks by soff (to 0 past the end), so a lane
// whose row lies past the tensor's span reads zeros instead of the memory that follows it. The
// arithmetic is scalar (SALU): soff passes through readfirstlane.
struct BufDesc {
  uint32_t w[4];
};
__device__ inline BufDesc make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return BufDesc{{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, kRsrcWord3}};
}
// The descriptor of the same tensor seen from byte offset off (wave-uniform): base + off and
// max(bytes - off, 0) addressable bytes.
__device__ inline BufDesc desc_at(const BufDesc& d, uint32_t off) {
  off = __builtin_amdgcn_readfirstlane(off);
  const uint64_t a = (((uint64_t)(d.w[1] & 0xFFFFu) << 32) | d.w[0]) + off;
  // max(bytes, off) - off on the scalar unit (written as a select, the compiler picks a clamped
  // vector subtract and a readfirstlane). s_max_u32 writes SCC: the clobber keeps the compiler
  // from placing it inside a carry chain (between the s_add_u32 and s_addc_u32 of the base
  // address above), where it would corrupt the carry into the high address bits.
  uint32_t hi;
  asm("s_max_u32 %0, %1, %2" : "=s"(hi) : "s"(d.w[2]), "s"(off) : "scc");
  const uint32_t n = hi - off;
  auto u = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane(x); };
  return BufDesc{{u((uint32_t)a), u((d.w[1] & 0xFFFF0000u) | ((uint32_t)(a >> 32) & 0xFFFFu)), u(n), d.w[3]}};
}
__device__ inline void dma16(const BufDesc& d0, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const BufDesc d = desc_at(d0, soff);
  const u32x4 rs = u32x4{d.w[0], d.w[1], d.w[2], d.w[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}
// The 4-byte form: lane l's 4 bytes land at LDS byte address lds_addr + 4 * l.
__device__ inline void dma4(const BufDesc& d0, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const BufDesc d = desc_at(d0, soff);
  const u32x4 rs = u32x4{d.w[0], d.w[1], d.w[2], d.w[3]};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}
// LDS reads addressed by 32-bit LDS byte addresses. Going through an integer address (instead of a
// generic pointer) lets the compiler put constant displacements into the instruction's offset field
// instead of recomputing each address with vector adds.
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ inline i32x4 lds_read_b128(uint32_t addr) { return *(const lds_i32x4*)(uintptr_t)addr; }
__device__ inline void lds_write_b64(uint32_t addr, i32x2 v) { *(lds_i32x2*)(uintptr_t)addr = v; }
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
