// fa_kernels.hpp — kernel arguments and launch entry points shared by the C ABI and the kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fa {

// Everything one launch needs; passed by value as the kernel argument.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;            // may be null
  int B, Nq, Nk, Hq, Hkv, group;  // group = Hq / Hkv
  int causal, wl, wr;
  int num_q_tiles;
  int64_t q_b, q_n, q_h;  // element strides
  int64_t k_b, k_n, k_h;
  int64_t v_b, v_n, v_h;
  int64_t o_b, o_n, o_h;
  uint32_t q_bytes, k_bytes, v_bytes, o_bytes;  // one head's addressable span, in bytes
  float scale_log2;      // softmax_scale * log2(e)   (times dq * dk for fp8)
  float out_scale;       // 1, or dv for fp8
};

// Backward pass: one launch of each of three kernels (delta, dq, dk/dv).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;          // [2, B, Hq, Nq] workspace: -rowsum(dout * out), then -lse / scale
                         // (-inf for rows with no admitted key)
  int B, Nq, Nk, Hq, Hkv, group;
  int causal, wl, wr;
  int num_q_tiles;       // of the dq kernel's query tiles
  int num_k_tiles;       // of the dk/dv kernel's key tiles
  int n_split;           // dk/dv workgroups per (K/V head, key tile), each for group / n_split query heads
  float* part;           // n_split > 1: fp32 partial dk, then dv, [n_split, B, Hkv, Nk, D] each
  int64_t q_b, q_n, q_h, k_b, k_n, k_h, v_b, v_n, v_h, o_b, o_n, o_h;
  int64_t do_b, do_n, do_h, dq_b, dq_n, dq_h, dk_b, dk_n, dk_h, dv_b, dv_n, dv_h;
  uint32_t q_bytes, k_bytes, v_bytes, o_bytes, do_bytes, dq_bytes, dk_bytes, dv_bytes;
  float scale;           // softmax_scale
  float scale_log2;      // softmax_scale * log2(e)
};

constexpr int kBwdQRows = 128;   // query rows per dq workgroup
constexpr int kBwdKRows = 128;   // keys per dk/dv workgroup
hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream);

// Tile shapes of the launch for head dimension D and storage type.
struct TileShape {
  int block_m, block_n, waves, lds_bytes;
};

TileShape tile_shape(int D, int dtype);
hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, int64_t grid, hipStream_t stream);

}  // namespace fa
