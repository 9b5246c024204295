// fa_fwd_f16.hip — FlashAttention forward for fp16 / bf16 storage on gfx950 (MI355X).
//
// The method ("What FlashAttention is and how it speeds up attention", sections 1-2): blocks of
// Q, K and V are staged in fast on-chip memory, attention is computed block by block inside it,
// and the output is updated with a running renormalisation, so the score matrix never reaches
// HBM; matmul, softmax and matmul are one kernel. The result is the exact softmax attention of
// "Flash Attention - Fast Memory-Efficient Attention" (skill page, Workflow 1 Step 2), with the
// causal / window / MQA-GQA options of its Workflow 2.
//
// Mapping onto CDNA4:
//  * One workgroup per (batch, query head, tile of BM = 32 * WAVES query rows); each 64-lane
//    wave owns 32 query rows. The grid is remapped so that the workgroups one XCD receives
//    (hardware deals blocks round-robin over the 8 XCDs) cover whole heads: a head's K/V stays
//    in that XCD's L2. Under a causal mask a head's heaviest query tiles start first.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{f16,bf16}: K rows
//    are the A operand (read from LDS), Q rows the B operand (kept in registers). In the 32x32
//    accumulator, lane l holds query l % 32 and 16 of the 32 keys; lanes l and l ^ 32 share a
//    query. The running max / sum of a query are therefore per-lane scalars, and a row
//    reduction is 16 in-register steps plus one v_permlane32_swap.
//  * O^T = V^T P^T reuses that accumulator as the B operand directly: the P values a lane
//    holds are a permutation of 8 consecutive MFMA k-slots, and V^T is read in the same
//    permuted key order with ds_read_b64_tr_b16 (LDS transpose read), so P never leaves
//    registers.
//  * K and V tiles (BN keys) are double-buffered in LDS: tile t+1 is fetched from HBM with
//    128-bit buffer loads while tile t is computed, then written to the other buffer. K rows are
//    XOR-swizzled by (row & 7) in 16-byte chunks and V rows by 2 * (row & 3), which keeps the
//    128-bit K reads and the transpose reads of V free of bank conflicts.
//  * Softmax in base 2: t = s * (scale * log2 e); p = exp2(t - m); alpha = exp2(m_old - m_new).
//  * Tiles with no admitted key are skipped; tiles admitted for every pair run without a mask;
//    only partial tiles (the causal diagonal, window edges, the ragged end) are masked.
//  * Ragged sizes: buffer resources bound each head's span, so loads past it return 0 and
//    stores past it are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.hpp"
#include "fa_mask.hpp"

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr float kLn2 = 0.69314718055994530942f;

struct F16 {
  static constexpr int kDtype = 0;
  __device__ static inline f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  __device__ static inline uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
  }
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
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Block index -> logical block index, so that each XCD's share is one contiguous range.
__device__ inline int xcd_remap(int id, int n) {
  const int xcd = id & 7, k = id >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
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

template <class TR, int D, int BN, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) fa_fwd_kernel(FwdArgs a) {
  constexpr int NT = WAVES * 64;        // threads per workgroup
  constexpr int BM = WAVES * 32;        // query rows per workgroup
  constexpr int ES = 2;                 // bytes per stored element
  constexpr int ROWB = D * ES;          // bytes per K/V row in LDS
  constexpr int TILEB = BN * ROWB;      // bytes per K (or V) tile
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int CH = BN * CPR / NT;     // chunks each thread moves per tile, per tensor
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int DB = D / 32;            // 32-wide column blocks of the output
  constexpr int KS = D / 16;            // MFMA k-steps over the head dimension
  static_assert(BN * CPR % NT == 0, "tile must split evenly over the workgroup");
  static_assert(CPR >= 8, "swizzles need at least 8 chunks per row");

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILEB];  // [stage][K | V][BN][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;      // half of the wave: which 16 of a block's 32 keys / k-slots
  const int l32 = lane & 31;     // query column of this lane inside the wave's 32 rows

  // ---- which (batch, head, query tile) this workgroup computes
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.num_q_tiles;
  int qt = L - bh * a.num_q_tiles;
  if (a.causal) qt = a.num_q_tiles - 1 - qt;     // heaviest tiles of a head first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int hk = h / a.group;                    // MQA/GQA: K/V head of this query head
  const int q0 = qt * BM;

  const MaskSpec ms{a.Nq, a.Nk, a.causal, a.wl, a.wr};

  const char* qb = (const char*)a.q + (b * a.q_b + h * a.q_h) * ES;
  const char* kbp = (const char*)a.k + (b * a.k_b + hk * a.k_h) * ES;
  const char* vbp = (const char*)a.v + (b * a.v_b + hk * a.v_h) * ES;
  char* ob = (char*)a.o + (b * a.o_b + h * a.o_h) * ES;
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc(qb, a.q_bytes);
  const __amdgpu_buffer_rsrc_t k_r = make_rsrc(kbp, a.k_bytes);
  const __amdgpu_buffer_rsrc_t v_r = make_rsrc(vbp, a.v_bytes);
  const __amdgpu_buffer_rsrc_t o_r = make_rsrc(ob, a.o_bytes);
  const uint32_t q_rowb = (uint32_t)(a.q_n * ES), k_rowb = (uint32_t)(a.k_n * ES);
  const uint32_t v_rowb = (uint32_t)(a.v_n * ES), o_rowb = (uint32_t)(a.o_n * ES);

  // ---- K/V tiles this workgroup visits, and this wave's rows
  const int wg_last = min(q0 + BM, a.Nq) - 1;
  int tb, te;
  tile_range(ms, q0, wg_last, BN, &tb, &te);
  const int w0 = q0 + wave * 32;
  const bool wave_live = w0 < a.Nq;
  const int w1 = min(w0 + 31, a.Nq - 1);
  const int my_row = w0 + l32;
  const int lo_i = (int)key_lo(ms, my_row);
  const int hi_i = (int)key_hi(ms, my_row);
  const uint32_t span_i = hi_i >= lo_i ? (uint32_t)(hi_i - lo_i + 1) : 0u;

  // ---- Q operands (B operand of S^T): row my_row, head-dim slots ks*16 + hl*8 .. +7
  i32x4 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qop[ks] = __builtin_amdgcn_raw_buffer_load_b128(q_r, (uint32_t)my_row * q_rowb + (ks * 16 + hl * 8) * ES, 0, 0);

  // ---- global -> register -> LDS staging of one K/V tile
  i32x4 kreg[CH], vreg[CH];
  auto gload = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT, row = c / CPR, cc = c % CPR;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(k_r, (uint32_t)(j0 + row) * k_rowb + cc * 16, 0, 0);
      vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(v_r, (uint32_t)(j0 + row) * v_rowb + cc * 16, 0, 0);
    }
  };
  auto lstore = [&](int st) {
    char* ks = smem + st * 2 * TILEB;
    char* vs = ks + TILEB;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT, row = c / CPR, cc = c % CPR;
      *(i32x4*)(ks + row * ROWB + ((cc ^ (row & 7)) << 4)) = kreg[i];
      *(i32x4*)(vs + row * ROWB + ((cc ^ ((row & 3) << 1)) << 4)) = vreg[i];
    }
  };

  // Per-lane LDS offsets. K (A operand of S^T): row kb*32 + l32, chunk (2*ks + hl) ^ (l32 & 7).
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + hl) ^ (l32 & 7)) << 4);
  // V (A operand of O^T, transpose read): within each 16-lane group g, source lane 4t + c reads
  // row 4*(g>>1) + t (+8 for the second read), columns db*32 + (g&1)*16 + 4c .. +3.
  const int g16 = lane >> 4, s16 = lane & 15, tr = s16 >> 2, tc = s16 & 3;
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = db * 4 + (g16 & 1) * 2 + (tc >> 1);
    voff[db] = (4 * (g16 >> 1) + tr) * ROWB + ((chunk ^ (tr << 1)) << 4) + (tc & 1) * 8;
  }

  const float c2 = a.scale_log2;
  float m = -INFINITY;   // running max of score * c2 for this lane's query
  float l = 0.f;         // this lane's share of the running sum (lanes l, l^32 split the keys)
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  if (tb < te) {
    gload(tb);
    lstore(0);
  }
  __syncthreads();

  for (int t = tb; t < te; ++t) {
    const int st = (t - tb) & 1;
    if (t + 1 < te) gload(t + 1);
    const int j0 = t * BN;
    const int cls = wave_live ? classify_tile(ms, w0, w1, j0, BN) : TILE_SKIP;
    if (cls != TILE_SKIP) {
      const char* ks = smem + st * 2 * TILEB;
      const char* vs = ks + TILEB;
      // S^T = K Q^T
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const i32x4 kop = *(const i32x4*)(ks + kb * 32 * ROWB + koff[k]);
          s[kb] = TR::mfma(kop, qop[k], s[kb]);
        }
      }
      // mask: key of accumulator r in block kb is j0 + kb*32 + (r/4)*8 + hl*4 + r%4
      if (cls == TILE_PARTIAL) {
        const int jl = j0 + hl * 4 - lo_i;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = jl + kb * 32 + (r >> 2) * 8 + (r & 3);
            if ((uint32_t)j >= span_i) s[kb][r] = -INFINITY;
          }
      }
      // online softmax (base 2)
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m, mx * c2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float rs = 0.f;
      uint32_t pk[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c2, -m_use));
          rs += p0 + p1;
          pk[kb][r >> 1] = TR::pack(p0, p1);
        }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const i32x4 pop = i32x4{(int)pk[kb][4 * half + 0], (int)pk[kb][4 * half + 1], (int)pk[kb][4 * half + 2],
                                  (int)pk[kb][4 * half + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const char* p = vs + (kb * 32 + half * 16) * ROWB + voff[db];
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * ROWB));
            const i32x4 vop = i32x4{__builtin_bit_cast(i32x2, v0)[0], __builtin_bit_cast(i32x2, v0)[1],
                                    __builtin_bit_cast(i32x2, v1)[0], __builtin_bit_cast(i32x2, v1)[1]};
            o[db] = TR::mfma(vop, pop, o[db]);
          }
        }
    }
    if (t + 1 < te) lstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2
  if (!wave_live || my_row >= a.Nq) return;
  const float l_tot = pair_sum(l);
  const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t w0v = TR::pack(o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv);
      const uint32_t w1v = TR::pack(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)w0v, (int)w1v}, o_r,
                                            (uint32_t)my_row * o_rowb + (db * 32 + q4 * 8 + hl * 4) * ES, 0, 0);
    }
  if (a.lse != nullptr && hl == 0) {
    const float lse = l_tot > 0.f ? (m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    a.lse[((int64_t)b * a.Hq + h) * a.Nq + my_row] = lse;
  }
}

template <class TR, int D>
static hipError_t launch_t(const FwdArgs& a, int64_t grid, hipStream_t stream) {
  constexpr int BN = 64, WAVES = 4;
  hipLaunchKernelGGL((fa_fwd_kernel<TR, D, BN, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_f16(const FwdArgs& a, int D, int dtype, int64_t grid, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_t<F16, 64>(a, grid, stream) : launch_t<F16, 128>(a, grid, stream);
  return D == 64 ? launch_t<BF16, 64>(a, grid, stream) : launch_t<BF16, 128>(a, grid, stream);
}

}  // namespace fa
