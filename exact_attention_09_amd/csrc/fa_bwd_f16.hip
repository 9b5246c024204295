// fa_bwd_f16.hip — FlashAttention backward pass for fp16 / bf16 on gfx950 (MI355X).
//
// The method recomputes attention from the saved log-sum-exp instead of storing the score
// matrix ("Flash Attention - Fast Memory-Efficient Attention", skill page, Quick start: IO-aware
// tiling and recomputation). For an upstream gradient dout of the output, with
// p_ij = exp(s_ij - lse_i), s = scale * q.k over admitted pairs:
//     dv_j = sum_i p_ij dout_i                 dp_ij = dout_i . v_j
//     ds_ij = p_ij (dp_ij - delta_i),          delta_i = dout_i . out_i  (= sum_j p_ij dp_ij)
//     dq_i = scale sum_j ds_ij k_j             dk_j = scale sum_i ds_ij q_i
// and a K/V head shared by several query heads (MQA/GQA) receives the sum of their terms.
//
// Two kernels, none with atomics (the result is deterministic), run in this order:
//  * dq: one workgroup per (batch, query head, 128 query rows), walking the K/V tiles the rows
//    attend to. Lanes own queries, as in the forward kernel: S^T = K Q^T and dP^T = V dO^T come
//    out with one query per lane, so lse_i and delta_i are per-lane scalars, and dS^T is the B
//    operand of dQ^T = K^T dS^T with K^T read by ds_read_b64_tr_b16 in the matching key order.
//    Each lane computes its row's delta from the dout values it holds and the same values of out,
//    and writes -delta and -lse / scale into a caller-provided fp32 workspace;
//  * dk/dv: one workgroup per (batch, K/V head, 128 keys), walking the query tiles (of every
//    query head that reads this K/V head) that attend to its keys. Lanes own keys: S = Q K^T and
//    dP = dO V^T come out with one key per lane; P and dS are the B operands of
//    dV^T = dO^T P and dK^T = Q^T dS, with dO^T and Q^T read by transpose reads.
// Tiles stream HBM -> LDS by 128-bit LDS-direct loads into rings of three slots (two for the
// dq kernel at D = 128, where a third would leave room for one workgroup per CU instead of two):
// a step's loads are issued right after its barrier into the slot freed by the step before, so
// they have the rest of the ring to land, and one barrier per step both publishes the landed
// tile and frees the next slot. Every tile uses the row swizzle of the forward kernel's K tile
// (conflict-free row reads); transpose reads pick the swizzle of each 8-row group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_f16_common.hpp"
#include "fa_kernels.hpp"
#include "fa_mask.hpp"
#include "fa_tile.hpp"

namespace fa {

template <class TR>
__device__ inline void unpack2(uint32_t w, float& x, float& y) {
  if constexpr (TR::kDtype == 0) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    x = (float)h[0];
    y = (float)h[1];
  } else {
    x = __uint_as_float(w << 16);
    y = __uint_as_float(w & 0xFFFF0000u);
  }
}

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------------------------
template <class TR, int D>
__global__ void __launch_bounds__(256) fa_bwd_dq_kernel(BwdArgs a) {
  using T = OpTile<D>;
  constexpr int NT = 256, BM = kBwdQRows, BN = 64, ES = 2;
  constexpr int ROWB = T::ROWB, TILEB = T::TILEB, KS = T::KS, DB = T::DB, KB = BN / 32;
  constexpr int CH = BN * (D / 8) / NT;     // 16-byte loads per thread per tile
  constexpr int NSL = D == 64 ? 3 : 2;      // ring slots per tensor
  __shared__ __attribute__((aligned(16))) char smem[2 * NSL * TILEB];   // [K ring | V ring]
  char* const kring = smem;
  char* const vring = smem + NSL * TILEB;

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, h, qt;
  schedule_block(blockIdx.x, a.sched_q, &b, &h, &qt);
  const int hk = h / a.group;
  const int q0 = qt * BM;
  const MaskSpec ms{a.Nq, a.Nk, a.causal, a.wl, a.wr};

  const char* kbp = (const char*)a.k + (b * a.k_b + hk * a.k_h) * ES;
  const char* vbp = (const char*)a.v + (b * a.v_b + hk * a.v_h) * ES;
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc((const char*)a.q + (b * a.q_b + h * a.q_h) * ES, a.q_bytes);
  const __amdgpu_buffer_rsrc_t do_r = make_rsrc((const char*)a.dout + (b * a.do_b + h * a.do_h) * ES, a.do_bytes);
  const __amdgpu_buffer_rsrc_t o_r = make_rsrc((const char*)a.o + (b * a.o_b + h * a.o_h) * ES, a.o_bytes);
  const __amdgpu_buffer_rsrc_t dq_r = make_rsrc((char*)a.dq + (b * a.dq_b + h * a.dq_h) * ES, a.dq_bytes);
  const uint32_t k_rowb = (uint32_t)(a.k_n * ES), v_rowb = (uint32_t)(a.v_n * ES);

  const int wg_last = min(q0 + BM, a.Nq) - 1;
  int tb, te;
  tile_range(ms, q0, wg_last, BN, &tb, &te);
  const int w0 = q0 + wave * 32;
  const bool wave_live = w0 < a.Nq;
  const int w1 = min(w0 + 31, a.Nq - 1);
  auto clamp_key = [&](int64_t x) { return (int)(x < -1 ? -1 : (x > a.Nk ? a.Nk : x)); };
  const int wlo0 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w0)));
  const int wlo1 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w1)));
  const int whi0 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w0)));
  const int whi1 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w1)));
  const int my_row = w0 + l32;
  const int lo_i = clamp_key(key_lo(ms, my_row));
  const int hi_i = clamp_key(key_hi(ms, my_row));
  const uint32_t span_i = hi_i >= lo_i ? (uint32_t)(hi_i - lo_i + 1) : 0u;

  // this lane's query row: Q and dO as B operands (head-dim values ks*16 + hl*8 .. +7), and the
  // same values of out for delta
  i32x4 qop[KS], dop[KS], oop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = __builtin_amdgcn_raw_buffer_load_b128(q_r, (uint32_t)my_row * (uint32_t)(a.q_n * ES) + (ks * 16 + hl * 8) * ES, 0, 0);
    dop[ks] = __builtin_amdgcn_raw_buffer_load_b128(do_r, (uint32_t)my_row * (uint32_t)(a.do_n * ES) + (ks * 16 + hl * 8) * ES, 0, 0);
    oop[ks] = __builtin_amdgcn_raw_buffer_load_b128(o_r, (uint32_t)my_row * (uint32_t)(a.o_n * ES) + (ks * 16 + hl * 8) * ES, 0, 0);
  }
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Nq;
  const int64_t r = ((int64_t)b * a.Hq + h) * a.Nq + my_row;
  const float l_row = my_row < a.Nq ? a.lse[r] : -INFINITY;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  // delta = rowsum(dout * out): this lane's half of the head dimension, then its partner's (lane
  // l ^ 32 holds the other half of the row). It goes into the workspace with -lse / scale, for the
  // dk/dv kernel, which runs after this one.
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float o0, o1, d0, d1;
      unpack2<TR>((uint32_t)oop[ks][e], o0, o1);
      unpack2<TR>((uint32_t)dop[ks][e], d0, d1);
      dpart = __builtin_fmaf(o0, d0, __builtin_fmaf(o1, d1, dpart));
    }
  const float ndelta = -(dpart + __shfl_xor(dpart, 32));   // -delta; rows past the end: 0
  float lse2 = INFINITY;                // rows past the end or with no key: p = 0
  if (l_row > -INFINITY) lse2 = l_row * kLog2e;
  if (my_row < a.Nq && hl == 0) {
    a.delta[r] = ndelta;
    a.delta[nrows + r] = l_row > -INFINITY ? -l_row / a.scale : -INFINITY;
  }

  uint32_t kgoff[CH], vgoff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int pos = (i * NT + tid) * 16, row = pos / ROWB, pc = (pos % ROWB) / 16;
    kgoff[i] = (uint32_t)row * k_rowb + ((pc ^ T::swz(row)) << 4);
    vgoff[i] = (uint32_t)row * v_rowb + ((pc ^ T::swz(row)) << 4);
  }
  const BufDesc k_d = make_desc(kbp, a.k_bytes), v_d = make_desc(vbp, a.v_bytes);
  const uint32_t kring_a = lds_addr_of(kring), vring_a = lds_addr_of(vring);
  auto dma = [&](const BufDesc& d, const uint32_t* goff, uint32_t soff, uint32_t lds) {
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(d, goff[i], soff, lds + wave * 64 * 16 + i * NT * 16);
  };
  auto barrier_keep = [&](int pending) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (pending >= 2 * CH) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * CH));
    else __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = T::row_off(l32, ks, hl);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e8 = 0; e8 < 2; ++e8) toff[db][e8] = T::tr_off(lane, db, e8);

  const float c2 = a.scale_log2;
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

#pragma unroll
  for (int i = 0; i < NSL - 1; ++i)
    if (tb + i < te) {
      dma(k_d, kgoff, (uint32_t)((tb + i) * BN) * k_rowb, kring_a + i * TILEB);
      dma(v_d, vgoff, (uint32_t)((tb + i) * BN) * v_rowb, vring_a + i * TILEB);
    }
  uint32_t s = 0, sn = (NSL - 1) * TILEB;   // slots of tiles t and t + NSL - 1
  for (int t = tb; t < te; ++t) {
    // tile t landed (with three slots, tile t + 1's loads stay in flight) and every wave is done
    // with tile t - 1, whose slot tile t + NSL - 1 refills
    barrier_keep(NSL == 3 && t + 1 < te ? 2 * CH : 0);
    if (t + NSL - 1 < te) {
      dma(k_d, kgoff, (uint32_t)((t + NSL - 1) * BN) * k_rowb, kring_a + sn);
      dma(v_d, vgoff, (uint32_t)((t + NSL - 1) * BN) * v_rowb, vring_a + sn);
    }
    const bool live = wave_live && t * BN + BN - 1 >= wlo0 && t * BN <= whi1;
    if (live) {
      uint32_t kt_base[DB][2];
      tr_bases<D>(kring_a + s, toff, kt_base);
      f32x16 st[KB], dpt[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) st[kb] = dpt[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kbase = opaque_vbase(kring_a + s + roff[ks]);
        const uint32_t vbase = opaque_vbase(vring_a + s + roff[ks]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          st[kb] = TR::mfma(lds_read_b128(kbase + kb * 32 * ROWB), qop[ks], st[kb]);
          dpt[kb] = TR::mfma(lds_read_b128(vbase + kb * 32 * ROWB), dop[ks], dpt[kb]);
        }
      }
      if (!(wlo1 <= t * BN && t * BN + BN - 1 <= whi0)) {
        const int jl = t * BN + hl * 4 - lo_i;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = jl + kb * 32 + (r >> 2) * 8 + (r & 3);
            st[kb][r] = (uint32_t)j < span_i ? st[kb][r] : -INFINITY;
          }
      }
      // ds^T = p (dp^T - delta), packed to the MFMA type in accumulator order
      uint32_t dsk[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c2, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r + 1], c2, -lse2));
          dsk[kb][r >> 1] = TR::pack(p0 * (dpt[kb][r] + ndelta), p1 * (dpt[kb][r + 1] + ndelta));
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const i32x4 dsop = i32x4{(int)dsk[kb][4 * half + 0], (int)dsk[kb][4 * half + 1], (int)dsk[kb][4 * half + 2],
                                   (int)dsk[kb][4 * half + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) dq[db] = TR::mfma(tr_operand<D>(kt_base, kb, half, db), dsop, dq[db]);
        }
    }
    sn = s;
    s = s == (NSL - 1) * TILEB ? 0 : s + TILEB;
  }

  // dq leaves through LDS (as the forward's output): every wave is past its last read of the
  // rings after this barrier; each wave writes its 32 rows into a private region in the MFMA
  // layout (16-byte chunk c of row r at c ^ (r % CPR)) and stores them by whole rows; rows past
  // Nq are dropped by the buffer range check.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (!wave_live) return;
  constexpr int OROWB = D * ES, CPR = OROWB / 16, RPI = 1024 / OROWB;
  static_assert(4 * 32 * OROWB <= 2 * NSL * TILEB, "the output stage fits in the rings");
  const uint32_t stage = lds_addr_of(smem) + wave * 32 * OROWB;
  const uint32_t dq_rowb = (uint32_t)(a.dq_n * ES);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t w0v = TR::pack(dq[db][4 * q4 + 0] * a.scale, dq[db][4 * q4 + 1] * a.scale);
      const uint32_t w1v = TR::pack(dq[db][4 * q4 + 2] * a.scale, dq[db][4 * q4 + 3] * a.scale);
      lds_write_b64(stage + l32 * OROWB + (((db * 4 + q4) ^ (l32 % CPR)) << 4) + hl * 8, i32x2{(int)w0v, (int)w1v});
    }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the reads below follow the writes (one wave: in order)
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const i32x4 v = lds_read_b128(stage + r * OROWB + ((c ^ (r % CPR)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(v, dq_r, (uint32_t)(w0 + r) * dq_rowb + c * 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------------------------
// At D = 64 the kernel is built for three waves per SIMD (168 registers; three workgroups share a
// compute unit's LDS): the few values that do not fit are held in scratch across the step loop and
// read back for the epilogue only. Measured 1.7% faster than two waves per SIMD on causal
// [4, 4096, 32, 64] (2% slower without a mask). At D = 128 one wave per SIMD.
template <class TR, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1)))
fa_bwd_dkdv_kernel(BwdArgs a) {
  using T = OpTile<D>;
  constexpr int NT = 256, BKV = kBwdKRows, BQ = 64, ES = 2;
  constexpr int ROWB = T::ROWB, TILEB = T::TILEB, KS = T::KS, DB = T::DB, QB = BQ / 32;
  constexpr int CH = BQ * (D / 8) / NT;
  constexpr int NS = 2 * KS, ND = 4 * DB;   // products per 32-query block: S and dP, dV and dK
  __shared__ __attribute__((aligned(16))) char smem[6 * TILEB];   // [Q0 Q1 Q2 | dO0 dO1 dO2]
  char* const qring = smem;
  char* const dring = smem + 3 * TILEB;
  // -lse / scale and -delta of each slot's 64 query rows (256 bytes each: one 4-byte LDS-direct load
  // per wave, every wave writing the same values)
  __shared__ __attribute__((aligned(16))) char sbuf[3 * 2 * 256];

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (batch, K/V head, split of its query heads, key tile) in the forward kernel's launch order,
  // longest work first under a causal mask: there the first key tiles meet the most query tiles
  int b, hs, kt;
  schedule_block(blockIdx.x, a.sched_k, &b, &hs, &kt);
  kt = a.num_k_tiles - 1 - kt;
  const int hk = hs / a.n_split, sp = hs - hk * a.n_split;
  const int gq = a.group / a.n_split;   // query heads of this workgroup: hk * group + sp * gq + 0 .. gq-1
  const int k0 = kt * BKV;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;
  const MaskSpec ms{a.Nq, a.Nk, a.causal, a.wl, a.wr};

  const __amdgpu_buffer_rsrc_t k_r = make_rsrc((const char*)a.k + (b * a.k_b + hk * a.k_h) * ES, a.k_bytes);
  const __amdgpu_buffer_rsrc_t v_r = make_rsrc((const char*)a.v + (b * a.v_b + hk * a.v_h) * ES, a.v_bytes);
  const __amdgpu_buffer_rsrc_t dk_r = make_rsrc((char*)a.dk + (b * a.dk_b + hk * a.dk_h) * ES, a.dk_bytes);
  const __amdgpu_buffer_rsrc_t dv_r = make_rsrc((char*)a.dv + (b * a.dv_b + hk * a.dv_h) * ES, a.dv_bytes);

  // query rows that admit some key of this workgroup: [i_lo, i_hi]. Key j is admitted by row i
  // iff lo(i) <= j <= hi(i); both bounds grow with i, so these rows form an interval.
  const int k_last = min(k0 + BKV, a.Nk) - 1;
  int i_lo = a.Nq, i_hi = -1;
  {
    // smallest i with hi(i) >= k0, largest i with lo(i) <= k_last (binary searches)
    int lo = 0, hi = a.Nq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key_hi(ms, mid) >= k0) hi = mid; else lo = mid + 1;
    }
    i_lo = lo;
    lo = -1;
    hi = a.Nq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (key_lo(ms, mid) <= k_last) lo = mid; else hi = mid - 1;
    }
    i_hi = lo;
  }
  i_lo = __builtin_amdgcn_readfirstlane(i_lo);
  i_hi = __builtin_amdgcn_readfirstlane(i_hi);
  const int ub = i_lo <= i_hi ? i_lo / BQ : 0, ue = i_lo <= i_hi ? i_hi / BQ + 1 : 0;
  const int nu = ue - ub;                     // query tiles per query head
  const int nsteps = nu * gq;

  // this lane's key: K and V as B operands
  i32x4 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = __builtin_amdgcn_raw_buffer_load_b128(k_r, (uint32_t)my_key * (uint32_t)(a.k_n * ES) + (ks * 16 + hl * 8) * ES, 0, 0);
    vop[ks] = __builtin_amdgcn_raw_buffer_load_b128(v_r, (uint32_t)my_key * (uint32_t)(a.v_n * ES) + (ks * 16 + hl * 8) * ES, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Load i of a thread covers tile row i * RPL + tid * 16 / ROWB; RPL is a multiple of 16 rows,
  // which keep the swizzle, so the loads differ only by whole rows, carried in the scalar offset.
  constexpr int RPL = NT * 16 / ROWB;
  static_assert(RPL % 16 == 0, "loads of a thread keep the row swizzle");
  const uint32_t q_rowb = (uint32_t)(a.q_n * ES), do_rowb = (uint32_t)(a.do_n * ES);
  uint32_t qgoff, dgoff;
  {
    const int row = tid * 16 / ROWB, pc = (tid * 16 % ROWB) / 16;
    qgoff = (uint32_t)row * q_rowb + ((pc ^ T::swz(row)) << 4);
    dgoff = (uint32_t)row * do_rowb + ((pc ^ T::swz(row)) << 4);
  }
  const uint32_t qring_a = lds_addr_of(qring), dring_a = lds_addr_of(dring);
  auto dma = [&](const BufDesc& d, uint32_t goff, uint32_t rowb, uint32_t soff, uint32_t lds) {
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(d, goff, soff + (uint32_t)(i * RPL) * rowb, lds + wave * 64 * 16 + i * NT * 16);
  };
  // waits for this thread's loads older than the newest step's (2 CH + 2 of them), then meets
  // the other waves
  constexpr int PEND = 2 * CH + 2;
  static_assert(PEND < 16, "vmcnt immediate below");
  auto barrier_keep = [&](bool keep_newest) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (keep_newest) __builtin_amdgcn_s_waitcnt(0x0070 | PEND);
    else __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // Descriptors of query head hh's Q, dO and workspace rows (set when the steps reach a new head)
  BufDesc q_d, d_d, w_d, e_d;
  auto set_head = [&](int hh) {
    q_d = make_desc((const char*)a.q + (b * a.q_b + hh * a.q_h) * ES, a.q_bytes);
    d_d = make_desc((const char*)a.dout + (b * a.do_b + hh * a.do_h) * ES, a.do_bytes);
    const int64_t row0 = ((int64_t)b * a.Hq + hh) * a.Nq;
    w_d = make_desc(a.delta + (int64_t)a.B * a.Hq * a.Nq + row0, (uint32_t)a.Nq * 4u);
    e_d = make_desc(a.delta + row0, (uint32_t)a.Nq * 4u);
  };
  // Steps run over the group's query heads (outer) and the query tiles ub .. ue - 1 (inner).
  auto advance = [&](int& hh, int& u) {
    if (++u == ue) {
      u = ub;
      ++hh;
      set_head(hh);
    }
  };
  const uint32_t sbuf_a = lds_addr_of(sbuf);
  // loads of the step (query tile u of the head set_head last chose) into the ring slot at byte
  // offset `slot`: Q and dO tiles, and the tile's rows of both workspace halves (every wave loads those 64 values into
  // the same place: 2 loads, same count per wave)
  auto issue = [&](int u, uint32_t slot) {
    dma(q_d, qgoff, q_rowb, (uint32_t)(u * BQ) * q_rowb, qring_a + slot);
    dma(d_d, dgoff, do_rowb, (uint32_t)(u * BQ) * do_rowb, dring_a + slot);
    const uint32_t st = sbuf_a + (slot / TILEB) * 512u;
    dma4(w_d, lane * 4, (uint32_t)(u * BQ) * 4u, st);
    dma4(e_d, lane * 4, (uint32_t)(u * BQ) * 4u, st + 256);
  };
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = T::row_off(l32, ks, hl);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e8 = 0; e8 < 2; ++e8) toff[db][e8] = T::tr_off(lane, db, e8);

  // Query rows that admit some key of this wave, [sw_lo, sw_hi], and rows that admit all 32 of
  // its keys, [aw_lo, aw_hi] (empty when the wave's keys run past Nk). With off = Nk - Nq and
  // right = 0 under the causal mask (else window_right), row i admits key j iff
  // i >= j - off - right (no bound when right < 0) and i <= j - off + window_left (no bound when
  // window_left < 0); both bounds move by one row per key, so the rows that admit some key of
  // j0..j1 run from the lower bound of j0 to the upper bound of j1, and the rows that admit all of
  // them from the lower bound of j1 to the upper bound of j0.
  int sw_lo, sw_hi, aw_lo, aw_hi;
  {
    const int64_t off = (int64_t)a.Nk - a.Nq, right = a.causal ? 0 : a.wr;
    const int64_t j0 = kw0, j1 = min(kw0 + 31, a.Nk - 1), jf = (int64_t)kw0 + 31;
    auto clamp_row = [&](int64_t x) { return (int)(x < -64 ? -64 : (x > a.Nq ? a.Nq : x)); };
    sw_lo = right < 0 ? 0 : clamp_row(j0 - off - right);
    sw_hi = a.wl < 0 ? a.Nq - 1 : min(a.Nq - 1, clamp_row(j1 - off + a.wl));
    aw_lo = right < 0 ? 0 : clamp_row(jf - off - right);
    aw_hi = a.wl < 0 ? a.Nq - 1 : min(a.Nq - 1, clamp_row(j0 - off + a.wl));
    if (kw0 >= a.Nk) sw_lo = a.Nq;      // no key: every block is skipped
    if (jf >= a.Nk) aw_lo = a.Nq;       // ragged keys: no block is full
  }
  // The rows that admit this lane's key, [ilo_j, ilo_j + span_j) (by the same bounds, for one key)
  int ilo_j, span_j;
  {
    const int64_t off = (int64_t)a.Nk - a.Nq, right = a.causal ? 0 : a.wr;
    const int64_t lo = right < 0 ? 0 : (int64_t)my_key - off - right;
    const int64_t hi = a.wl < 0 ? (int64_t)a.Nq - 1 : (int64_t)my_key - off + a.wl;
    const int64_t lo_c = lo < 0 ? 0 : lo, hi_c = hi > a.Nq - 1 ? a.Nq - 1 : hi;
    ilo_j = (int)(lo_c > a.Nq ? a.Nq : lo_c);
    span_j = my_key < a.Nk && hi_c >= lo_c ? (int)(hi_c - lo_c + 1) : 0;
  }
  sw_lo = __builtin_amdgcn_readfirstlane(sw_lo);
  sw_hi = __builtin_amdgcn_readfirstlane(sw_hi);
  aw_lo = __builtin_amdgcn_readfirstlane(aw_lo);
  aw_hi = __builtin_amdgcn_readfirstlane(aw_hi);
  // this wave's keys against the 32-query block starting at row i0: none (0), some (1) or all (2)
  // of the pairs admitted
  auto block_class = [&](int i0) {
    if (i0 > sw_hi || i0 + 31 < sw_lo) return 0;
    if (i0 >= aw_lo && i0 + 31 <= aw_hi) return 2;
    return 1;
  };

  const float c2 = a.scale_log2;
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};

  int next_h = hk * a.group + sp * gq, next_u = ub;   // the next step to issue
  int u = ub;                                // query tile of the step being computed
  set_head(next_h);
  if (nsteps > 0) {
    issue(next_u, 0);
    advance(next_h, next_u);
  }
  if (nsteps > 1) {
    issue(next_u, TILEB);
    advance(next_h, next_u);
  }
  uint32_t s = 0, s2 = 2 * TILEB;            // slots of steps n and n + 2
  for (int n = 0; n < nsteps; ++n) {
    const bool more = n + 1 < nsteps;
    // step n's loads landed (step n + 1's stay in flight) and every wave is done with step n - 1,
    // whose slot step n + 2 refills
    barrier_keep(more);
    if (n + 2 < nsteps) {
      issue(next_u, s2);
      advance(next_h, next_u);
    }
    const uint32_t st = sbuf_a + (s / TILEB) * 512u;
    uint32_t qt_base[DB][2], dt_base[DB][2], qr[KS], dr[KS];
    tr_bases<D>(qring_a + s, toff, qt_base);
    tr_bases<D>(dring_a + s, toff, dt_base);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[ks] = opaque_vbase(qring_a + s + roff[ks]);
      dr[ks] = opaque_vbase(dring_a + s + roff[ks]);
    }
    // Accumulators of block qb start from the rows' offsets: S from -lse / scale (so that
    // p = 2^(S * scale * log2 e)), dP from -delta (so that ds = p * dP). Accumulator r holds query
    // i0 + (r/4)*8 + hl*4 + r%4: four groups of four consecutive rows, one 16-byte read each.
    auto init_acc = [&](int qb, f32x16& sc, f32x16& dp) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t at = st + (uint32_t)(qb * 32 + g * 8 + hl * 4) * 4u;
        const i32x4 wv = lds_read_b128(at), nv = lds_read_b128(at + 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[g * 4 + e] = __int_as_float(wv[e]);
          dp[g * 4 + e] = __int_as_float(nv[e]);
        }
      }
    };
    // Operand and product m of block qb's sequences. S/dP (NS of them): k-slot m / 2, even m
    // S += Q K^T, odd m dP += dO V^T. dV/dK (ND of them): half m / (2 DB), column block
    // (m / 2) % DB, even m dV^T += dO^T P, odd m dK^T += Q^T dS.
    auto sdp_operand = [&](int qb, int m) { return lds_read_b128((m % 2 ? dr : qr)[m / 2] + qb * 32 * ROWB); };
    auto sdp_mfma = [&](int m, const i32x4& x, f32x16& sc, f32x16& dp) {
      if (m % 2 == 0) sc = TR::mfma(x, kop[m / 2], sc);
      else dp = TR::mfma(x, vop[m / 2], dp);
    };
    auto dvdk_operand = [&](int qb, int m) {
      return tr_operand<D>(m % 2 ? qt_base : dt_base, qb, m / (2 * DB), (m / 2) % DB);
    };
    auto dvdk_mfma = [&](int m, const i32x4& x, const uint32_t (&pk)[8], const uint32_t (&dsk)[8]) {
      const int h4 = 4 * (m / (2 * DB)), db = (m / 2) % DB;
      if (m % 2 == 0) dv[db] = TR::mfma(x, i32x4{(int)pk[h4], (int)pk[h4 + 1], (int)pk[h4 + 2], (int)pk[h4 + 3]}, dv[db]);
      else dk[db] = TR::mfma(x, i32x4{(int)dsk[h4], (int)dsk[h4 + 1], (int)dsk[h4 + 2], (int)dsk[h4 + 3]}, dk[db]);
    };
    // softmax pair pi of a block: p = 2^(S c2), ds = p dP, both packed to the MFMA type
    auto pair = [&](const f32x16& sc, const f32x16& dp, int pi, uint32_t (&pk)[8], uint32_t (&dsk)[8]) {
      const float p0 = __builtin_amdgcn_exp2f(sc[2 * pi] * c2), p1 = __builtin_amdgcn_exp2f(sc[2 * pi + 1] * c2);
      pk[pi] = TR::pack(p0, p1);
      dsk[pi] = TR::pack(p0 * dp[2 * pi], p1 * dp[2 * pi + 1]);
    };

    const int i0 = u * BQ;
    const int c0 = __builtin_amdgcn_readfirstlane(block_class(i0));
    const int c1 = __builtin_amdgcn_readfirstlane(block_class(i0 + 32));
    if (D == 128 && c0 == 2 && c1 == 2) {
      // Both blocks full: one sequence S/dP(0), S/dP(1), dV/dK(0), dV/dK(1) in which the softmax
      // of block 0 runs beside S/dP(1) and that of block 1 beside dV/dK(0). Operands are read
      // PF products ahead. At D = 128 the kernel runs one wave per SIMD, and this overlap within
      // the wave measured 8% faster; at D = 64 three waves share each SIMD and overlap each
      // other, and the sequence (252 registers: two waves per SIMD) measured 6% slower.
      constexpr int NE = 2 * (NS + ND), PF = 2, GS = NS / 8, GD = ND / 8;
      f32x16 sc0, dp0, sc1, dp1;
      uint32_t pk0[8], dsk0[8], pk1[8], dsk1[8];
      i32x4 opnd[NE];
      auto read_op = [&](int e) {
        if (e < NS) opnd[e] = sdp_operand(0, e);
        else if (e < 2 * NS) opnd[e] = sdp_operand(1, e - NS);
        else if (e < 2 * NS + ND) opnd[e] = dvdk_operand(0, e - 2 * NS);
        else opnd[e] = dvdk_operand(1, e - 2 * NS - ND);
      };
      init_acc(0, sc0, dp0);
      init_acc(1, sc1, dp1);
#pragma unroll
      for (int e = 0; e < PF; ++e) read_op(e);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NE>([&](auto E) {
        constexpr int e = decltype(E)::value;
        if constexpr (e + PF < NE) read_op(e + PF);
        if (e < NS) {
          sdp_mfma(e, opnd[e], sc0, dp0);
        } else if (e < 2 * NS) {
          sdp_mfma(e - NS, opnd[e], sc1, dp1);
          if ((e - NS) % GS == GS - 1) {
            const int pi = (e - NS) / GS;
            pair(sc0, dp0, pi, pk0, dsk0);
            asm volatile("" ::"v"(pk0[pi]), "v"(dsk0[pi]));
          }
        } else if (e < 2 * NS + ND) {
          dvdk_mfma(e - 2 * NS, opnd[e], pk0, dsk0);
          if ((e - 2 * NS) % GD == GD - 1) {
            const int pi = (e - 2 * NS) / GD;
            pair(sc1, dp1, pi, pk1, dsk1);
            asm volatile("" ::"v"(pk1[pi]), "v"(dsk1[pi]));
          }
        } else {
          dvdk_mfma(e - 2 * NS - ND, opnd[e], pk1, dsk1);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int cls = qb == 0 ? c0 : c1;
        if (cls == 0) continue;
        f32x16 sc, dp;
        init_acc(qb, sc, dp);
#pragma unroll
        for (int m = 0; m < NS; ++m) sdp_mfma(m, sdp_operand(qb, m), sc, dp);
        if (cls == 1) {
          const int il = i0 + qb * 32 + hl * 4 - ilo_j;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = il + (r >> 2) * 8 + (r & 3);
            sc[r] = (uint32_t)i < (uint32_t)span_j ? sc[r] : -INFINITY;
          }
        }
        uint32_t pk[8], dsk[8];
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) pair(sc, dp, pi, pk, dsk);
#pragma unroll
        for (int m = 0; m < ND; ++m) dvdk_mfma(m, dvdk_operand(qb, m), pk, dsk);
      }
    }
    if (++u == ue) u = ub;
    s2 = s;
    s = s == 2 * TILEB ? 0 : s + TILEB;
  }

  if (a.n_split > 1) {
    if (my_key >= a.Nk) return;
    // fp32 partial sums; fa_bwd_reduce_kernel adds the splits and scales dk
    const int64_t slab = (int64_t)a.n_split * a.B * a.Hkv * a.Nk * D;
    float* pk_row = a.part + ((((int64_t)sp * a.B + b) * a.Hkv + hk) * a.Nk + my_key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = db * 32 + q4 * 8 + hl * 4;
        *(f32x4*)(pk_row + col) = f32x4{dk[db][4 * q4], dk[db][4 * q4 + 1], dk[db][4 * q4 + 2], dk[db][4 * q4 + 3]};
        *(f32x4*)(pk_row + slab + col) = f32x4{dv[db][4 * q4], dv[db][4 * q4 + 1], dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]};
      }
    return;
  }
  // dk and dv leave through LDS (as the forward's output): every wave is past its last read of
  // the rings after this barrier; each wave writes its 32 keys' rows of dk, then dv, into a
  // private region and stores them by whole rows; keys past Nk are dropped by the buffer range
  // check. (n_split is uniform: every wave of a workgroup takes the same branch.)
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  constexpr int OROWB = D * ES, CPR = OROWB / 16, RPI = 1024 / OROWB;
  static_assert(4 * 2 * 32 * OROWB <= 6 * TILEB, "the output stage fits in the rings");
  const uint32_t stage_k = lds_addr_of(smem) + wave * 2 * 32 * OROWB, stage_v = stage_k + 32 * OROWB;
  const uint32_t dk_rowb = (uint32_t)(a.dk_n * ES), dv_rowb = (uint32_t)(a.dv_n * ES);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t k0v = TR::pack(dk[db][4 * q4 + 0] * a.scale, dk[db][4 * q4 + 1] * a.scale);
      const uint32_t k1v = TR::pack(dk[db][4 * q4 + 2] * a.scale, dk[db][4 * q4 + 3] * a.scale);
      const uint32_t v0v = TR::pack(dv[db][4 * q4 + 0], dv[db][4 * q4 + 1]);
      const uint32_t v1v = TR::pack(dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]);
      const uint32_t off = l32 * OROWB + (((db * 4 + q4) ^ (l32 % CPR)) << 4) + hl * 8;
      lds_write_b64(stage_k + off, i32x2{(int)k0v, (int)k1v});
      lds_write_b64(stage_v + off, i32x2{(int)v0v, (int)v1v});
    }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the reads below follow the writes (one wave: in order)
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const uint32_t so = r * OROWB + ((c ^ (r % CPR)) << 4);
    const i32x4 kv = lds_read_b128(stage_k + so), vv = lds_read_b128(stage_v + so);
    __builtin_amdgcn_raw_buffer_store_b128(kv, dk_r, (uint32_t)(kw0 + r) * dk_rowb + c * 16, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(vv, dv_r, (uint32_t)(kw0 + r) * dv_rowb + c * 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------------------------
// dk, dv = the sum over the n_split query-head splits of the fp32 partials (in split order, so the
// result does not depend on timing), dk times softmax_scale; 4 columns per thread.
template <class TR, int D>
__global__ void __launch_bounds__(256) fa_bwd_reduce_kernel(BwdArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)a.B * a.Hkv * a.Nk * D;   // floats of one split
  if (gid * 4 >= per) return;
  const int64_t row = gid / (D / 4);
  const int col = (int)(gid - row * (D / 4)) * 4;
  const int key = (int)(row % a.Nk);
  const int64_t bh = row / a.Nk;
  const int hk = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
  f32x4 sk = f32x4{}, sv = f32x4{};
  const int64_t slab = (int64_t)a.n_split * per;
  for (int s = 0; s < a.n_split; ++s) {
    sk += *(const f32x4*)(a.part + s * per + gid * 4);
    sv += *(const f32x4*)(a.part + slab + s * per + gid * 4);
  }
  const uint32_t k0 = TR::pack(sk[0] * a.scale, sk[1] * a.scale), k1 = TR::pack(sk[2] * a.scale, sk[3] * a.scale);
  const uint32_t v0 = TR::pack(sv[0], sv[1]), v1 = TR::pack(sv[2], sv[3]);
  *(i32x2*)((char*)a.dk + (b * a.dk_b + (int64_t)key * a.dk_n + hk * a.dk_h + col) * 2) = i32x2{(int)k0, (int)k1};
  *(i32x2*)((char*)a.dv + (b * a.dv_b + (int64_t)key * a.dv_n + hk * a.dv_h + col) * 2) = i32x2{(int)v0, (int)v1};
}

// ---------------------------------------------------------------------------------------------
template <class TR, int D>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  // dq first: it also writes the workspace rows (-delta, -lse / scale) that dk/dv reads
  hipLaunchKernelGGL((fa_bwd_dq_kernel<TR, D>), dim3((unsigned)((int64_t)a.B * a.Hq * a.num_q_tiles)), dim3(256), 0,
                     stream, a);
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<TR, D>),
                     dim3((unsigned)((int64_t)a.B * a.Hkv * a.n_split * a.num_k_tiles)), dim3(256), 0, stream, a);
  if (a.n_split > 1) {
    const int64_t quads = (int64_t)a.B * a.Hkv * a.Nk * (D / 4);
    hipLaunchKernelGGL((fa_bwd_reduce_kernel<TR, D>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_bwd_t<F16, 64>(a, stream) : launch_bwd_t<F16, 128>(a, stream);
  return D == 64 ? launch_bwd_t<BF16, 64>(a, stream) : launch_bwd_t<BF16, 128>(a, stream);
}

}  // namespace fa
