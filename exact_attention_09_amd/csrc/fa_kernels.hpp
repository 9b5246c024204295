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

// Tile shapes of the launch for head dimension D and storage type.
struct TileShape {
  int block_m, block_n, waves, lds_bytes;
};

TileShape tile_shape(int D, int dtype);
hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, int64_t grid, hipStream_t stream);

}  // namespace fa
