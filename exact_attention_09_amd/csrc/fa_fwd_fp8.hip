// fa_fwd_fp8.hip — FlashAttention forward for fp8 e4m3 storage on gfx950 (MI355X).
//
// Same method and pipeline as the fp16/bf16 kernel (blocks of Q, K, V in on-chip memory, online
// softmax with a running renormalisation, one fused kernel: "What FlashAttention is and how it
// speeds up attention", sections 1-2), for the pages' fp8 inputs ("Flash Attention - Fast
// Memory-Efficient Attention", skill page, Workflow 3: q, k, v cast to float8_e4m3). q, k, v are
// e4m3 codes with per-tensor dequantisation scales dq, dk, dv; the score is
// softmax_scale * dq * dk * <q8, k8> and the output sum_j p_ij * dv * v8_j, written as bf16.
//
// CDNA4 mapping (differences from the 16-bit kernel):
//  * Both products run on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulate): a lane
//    holds 32 consecutive k-slots, so one MFMA covers 64 head-dim values of S^T = K Q^T, and one
//    covers 64 keys of O^T = V^T P^T.
//  * P is rounded to e4m3 after a 2^8 shift that keeps small weights above the format's
//    subnormal range. p * 2^8 must stay <= 448 (the largest e4m3 value). The exponentials of a
//    tile are taken against the reference m of the tiles before it, without the tile's row max;
//    only when a lane's sum of 2^8 p exceeds 448 (the one case in which a single term can) does
//    the wave take the row max, and m moves if that max exceeds it by more than 0.8 (log2 units),
//    to 4 above the max, with O and l rescaled and the tile's exponentials taken again. With the
//    row max at weight 2^(8 - 4) = 16, a lane's 32 keys rarely sum past 448. The running sum (and
//    so the lse) uses the unrounded fp32 p.
//  * V^T is read with ds_read_b64_tr_b8: a lane receives 8 consecutive LDS rows of one column.
//    The 16 keys a lane half holds in the S^T accumulator (keys g*8 + half*4 + e, g, e < 4, of
//    each 32-key block) are stored as 16 consecutive LDS rows (row half*16 + g*4 + e): the HBM ->
//    LDS loads pick the global row of each LDS row, so this permutation costs nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_mask.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// log2 of the 2^8 shift applied to p before its e4m3 rounding, and the reference threshold.
// When the reference moves it is placed kLift above the tile's max, so that p <= 2^-kLift right
// after the move and the next move needs a rise of kTau8 + kLift: fewer moves (each rescales O).
// kLift is a whole number, so the weight of the max itself, 2^(8 - kLift) after the shift, is an
// exact e4m3 value (as 2^8 was without the lift); weights down to 2^(-14 + kLift) of the row max
// stay in e4m3's normal range. A lane's sum of 2^8 p at most kSumBound8 = 448 bounds each term.
// (A lift of 2 would make that sum exceed 448 in about a quarter of the tiles of a random causal
// [4096, 64] head, 4 in about 3%, the share in which the reference is set or moves anyway.)
constexpr float kPShiftLog2 = 8.0f;
constexpr float kTau8 = 0.8f;
constexpr float kLift = 4.0f;
constexpr float kSumBound8 = 448.0f;

// 64-bank LDS swizzles (16-byte chunk XOR) for 64- and 128-byte rows.
template <int ROWB>
__device__ inline int k_swz8(int row) {
  return ROWB == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
}
template <int ROWB>
__device__ inline int v_swz8(int row) {
  return ROWB == 64 ? ((row >> 2) & 1) << 1 : ((row >> 1) & 3) << 1;
}
// Key (within the tile) stored at LDS row rho of a V tile.
__device__ inline int v_key_of_row(int rho) {
  return (rho & ~31) | (((rho >> 2) & 3) << 3) | (((rho >> 4) & 1) << 2) | (rho & 3);
}

// max(a, b, c) in one v_max3_f32. Written out because fmaxf makes the compiler canonicalise each
// MFMA result first (an extra v_max per input); the scores here are finite or -inf, never NaN.
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, int BN, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) fa_fwd_fp8_kernel(FwdArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * 32;
  constexpr int ROWB = D;               // one byte per element
  constexpr int TILEB = BN * ROWB;
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int CH = BN * CPR / NT;     // HBM -> LDS loads per thread per tile, per tensor
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int DB = D / 32;            // 32-wide output column blocks
  constexpr int KS = D / 64;            // MFMA k-steps over the head dimension
  constexpr int NS = 3;
  static_assert(BN == 64, "the P operand packs two 32-key blocks into one 64-key MFMA");
  static_assert(BN * CPR % NT == 0, "tile must split evenly over the workgroup");
  static_assert(ROWB == 64 || ROWB == 128, "swizzles are laid out for 64- or 128-byte rows");

  __shared__ __attribute__((aligned(16))) char smem[2 * NS * TILEB];  // [K0 K1 K2 | V0 V1 V2]
  char* const kring = smem;
  char* const vring = smem + NS * TILEB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // which (batch, head, query tile) this workgroup computes
  int b, h, qt;
  schedule_block(blockIdx.x, a.sched, &b, &h, &qt);
  const int hk = (int)fdiv((uint32_t)h, a.sched.group);
  const int q0 = qt * BM;
  const SeqView sv = seq_view(a, b, h, D, 1, 2);
  if (q0 >= sv.Nq) return;                       // past the end of a shorter packed sequence

  const MaskSpec ms{sv.Nq, sv.Nk, a.causal, a.wl, a.wr};

  const char* qb = (const char*)a.q + (sv.q0 + h * a.q_h);
  const char* kbp = (const char*)a.k + (sv.k0 + hk * a.k_h);
  const char* vbp = (const char*)a.v + (sv.v0 + hk * a.v_h);
  char* ob = (char*)a.o + (sv.o0 + h * a.o_h) * 2;
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc(qb, sv.q_bytes);
  const __amdgpu_buffer_rsrc_t o_r = make_rsrc(ob, sv.o_bytes);
  const uint32_t q_rowb = (uint32_t)a.q_n, k_rowb = (uint32_t)a.k_n;
  const uint32_t v_rowb = (uint32_t)a.v_n, o_rowb = (uint32_t)(a.o_n * 2);

  const int wg_last = min(q0 + BM, sv.Nq) - 1;
  int tb, te;
  tile_range(ms, q0, wg_last, BN, &tb, &te);
  const int w0 = q0 + wave * 32;
  const bool wave_live = w0 < sv.Nq;
  const int w1 = min(w0 + 31, sv.Nq - 1);
  // tiles with an admitted key for some row of the wave: [jlo, jhi); for every row: [flo, fhi)
  auto clamp_key = [&](int64_t x) { return (int)(x < -1 ? -1 : (x > sv.Nk ? sv.Nk : x)); };
  const int wlo0 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w0)));
  const int wlo1 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w1)));
  const int whi0 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w0)));
  const int whi1 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w1)));
  int jlo = 0, jhi = 0;
  if (wave_live && whi1 >= wlo0) {
    jlo = max(tb, wlo0 / BN);
    jhi = min(te, whi1 / BN + 1);
  }
  const int flo = (wlo1 + BN - 1) / BN, fhi = (whi0 + 1) / BN;
  const int my_row = w0 + l32;
  const int lo_i = clamp_key(key_lo(ms, my_row));
  const int hi_i = clamp_key(key_hi(ms, my_row));
  const uint32_t span_i = hi_i >= lo_i ? (uint32_t)(hi_i - lo_i + 1) : 0u;

  // Q operands (B operand of S^T): row my_row, head-dim bytes ks*64 + hl*32 .. +31; loaded in
  // the prologue behind the first K/V tile loads
  i32x8 qop[KS];

  // HBM -> LDS: slot position P = (i * NT + tid) * 16 holds LDS row P / ROWB, physical chunk
  // (P % ROWB) / 16. K rows are in key order; V rows in the permuted order above.
  uint32_t kgoff[CH], vgoff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int pos = (i * NT + tid) * 16, row = pos / ROWB, pc = (pos % ROWB) / 16;
    kgoff[i] = (uint32_t)row * k_rowb + ((pc ^ k_swz8<ROWB>(row)) << 4);
    vgoff[i] = (uint32_t)v_key_of_row(row) * v_rowb + ((pc ^ v_swz8<ROWB>(row)) << 4);
  }
  const BufDesc k_d = make_desc(kbp, sv.k_bytes), v_d = make_desc(vbp, sv.v_bytes);
  const uint32_t kring_a = lds_addr_of(kring), vring_a = lds_addr_of(vring);
  auto dma = [&](const BufDesc& d, const uint32_t* goff, uint32_t soff, uint32_t lds) {
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(d, goff[i], soff, lds + wave * 64 * 16 + i * NT * 16);
  };
  auto barrier_keep = [&](int pending) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (pending >= 2 * CH) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * CH));
    else if (pending >= CH) __builtin_amdgcn_s_waitcnt(0x0070 | CH);
    else __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // K (A operand of S^T): row kb*32 + l32, bytes ks*64 + hl*32 .. +31 = chunks ks*4 + hl*2 + {0,1}
  int koff[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int part = 0; part < 2; ++part)
      koff[ks][part] = l32 * ROWB + (((ks * 4 + hl * 2 + part) ^ k_swz8<ROWB>(l32)) << 4);
  // V (A operand of O^T, ds_read_b64_tr_b8): in 16-lane group g, source lane 2r + c reads LDS
  // row (g>>1)*16 + r (+ kb*32 + part*8), bytes db*32 + (g&1)*16 + 8c .. +7.
  const int g16 = lane >> 4, s16 = lane & 15, tr8 = s16 >> 1, tc8 = s16 & 1;
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = db * 2 + (g16 & 1);
    voff[db] = ((g16 >> 1) * 16 + tr8) * ROWB + ((chunk ^ v_swz8<ROWB>(tr8)) << 4) + tc8 * 8;
  }

  const float c2 = a.scale_log2;
  // Reference of score * c2, starting at a huge negative finite value (a fully masked tile then
  // gives p = 0 with no special case; the first admitted key moves it).
  float m = -1e30f;
  float l = 0.f;         // sum of 2^8 * p over this lane's keys
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  // S MFMA e (k-step e / KB, key block e % KB) and its K operand (two 16-byte LDS reads)
  auto k_operand = [&](uint32_t slot, int e) {
    const int k = e / KB, kb = e % KB;
    const i32x4 x0 = lds_read_b128(opaque_vbase(slot + koff[k][0]) + kb * 32 * ROWB);
    const i32x4 x1 = lds_read_b128(opaque_vbase(slot + koff[k][1]) + kb * 32 * ROWB);
    return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  // V^T operand of column block db: 8 LDS rows per transpose read, 4 reads = the tile's 64 keys
  auto v_operand = [&](uint32_t slot, int db) {
    const uint32_t vbase = opaque_vbase(slot + voff[db]);
    i32x2 part[4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) part[kb * 2 + pr] = lds_read_tr8(vbase + (kb * 32 + pr * 8) * ROWB);
    return i32x8{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
  };
  constexpr int NSM = KS * KB;          // S MFMAs per tile
  auto mask_tile = [&](f32x16 (&sc)[KB], int t) {
    const int jl = t * BN + hl * 4 - lo_i;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jl + kb * 32 + (r >> 2) * 8 + (r & 3);
        sc[kb][r] = (uint32_t)j < span_i ? sc[kb][r] : -INFINITY;
      }
  };

  // ---- software pipeline, as in the 16-bit kernel: step j issues the loads of K(j+3) and V(j+1),
  // runs PV(j-1) and S(j+1) on the matrix pipe and the softmax of tile j on the vector pipe
  // (against the reference of the tiles before it, checked afterwards by the lanes' sums).
  // r0, r1, r2: byte offsets of ring slots (j - tb) % 3, +1, +2.
  const int need_lo = jlo - 1;
  const uint32_t need_n = jlo < jhi ? (uint32_t)(jhi - jlo + 2) : 0u;
  const uint32_t full_n = fhi > flo ? (uint32_t)(fhi - flo) : 0u;
  uint32_t r0 = 0, r1 = TILEB, r2 = 2 * TILEB;
  uint32_t k_soff = (uint32_t)((tb + 3) * BN) * k_rowb;
  uint32_t v_soff = (uint32_t)((tb + 1) * BN) * v_rowb;

  // V slot 2 stands for V(tb-1), read against P = 0 by the first step: zero it
#pragma unroll
  for (int c = tid * 16; c < TILEB; c += NT * 16) *(i32x4*)(vring + 2 * TILEB + c) = i32x4{};
  if (tb < te) {
    dma(k_d, kgoff, (uint32_t)(tb * BN) * k_rowb, kring_a);
    if (tb + 1 < te) dma(k_d, kgoff, (uint32_t)((tb + 1) * BN) * k_rowb, kring_a + TILEB);
    dma(v_d, vgoff, (uint32_t)(tb * BN) * v_rowb, vring_a);
    if (tb + 2 < te) dma(k_d, kgoff, (uint32_t)((tb + 2) * BN) * k_rowb, kring_a + 2 * TILEB);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_row * q_rowb + ks * 64 + hl * 32;
    const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(q_r, off, 0, 0);
    const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(q_r, off + 16, 0, 0);
    qop[ks] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q and the first tiles have landed
  barrier_keep(0);
  f32x16 sa[KB], sb[KB];
  int pa[8], pb[8];      // e4m3 codes of 2^8 p, in accumulator order (byte kb*16 + r)
#pragma unroll
  for (int w = 0; w < 8; ++w) pa[w] = pb[w] = 0;
  {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sa[kb] = f32x16{};
#pragma unroll
    for (int e = 0; e < NSM; ++e) sa[e % KB] = mfma_fp8(k_operand(kring_a, e), qop[e / KB], sa[e % KB]);
  }
  barrier_keep(0);   // every wave has read K(tb) before step tb refills its slot

  auto step = [&](int j, f32x16 (&sc)[KB], f32x16 (&sn)[KB], const int (&pp)[8], int (&pc)[8]) {
    const bool k3 = j + 3 < te, v1 = j + 1 < te;
    if (k3) dma(k_d, kgoff, k_soff, kring_a + r0);
    if (v1) dma(v_d, vgoff, v_soff, vring_a + r1);
    if ((uint32_t)(j - need_lo) < need_n) {
      if (!((uint32_t)(j - flo) < full_n)) mask_tile(sc, j);
      i32x8 vop[DB], kop[NSM];
#pragma unroll
      for (int db = 0; db < DB; ++db) vop[db] = v_operand(vring_a + r2, db);      // V(j-1)
#pragma unroll
      for (int e = 0; e < NSM; ++e) kop[e] = k_operand(kring_a + r1, e);         // K(j+1)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sn[kb] = f32x16{};
      const i32x8 pop = i32x8{pp[0], pp[1], pp[2], pp[3], pp[4], pp[5], pp[6], pp[7]};
      // 2^8 p = exp2(s c - m + 8) for the tile's code words wq (kb = wq / 4, w4 = wq % 4), against
      // the reference of the tiles before it; rs sums this lane's unrounded values (from -0, which
      // the first addition leaves out). The two conversions of a word write its low and high
      // halves, so the word's old value (codes of tile j - 2, read by the step before) is a free
      // first operand.
      float rs = -0.f;
      auto codes = [&](int wq, float shift) {
        const int kb = wq / 4, w4 = wq % 4;
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][4 * w4 + u], c2, shift));
        rs += (p[0] + p[1]) + (p[2] + p[3]);   // one dependent addition per word (c5: -2 to -4%)
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pc[wq], false);
        pc[wq] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        asm volatile("" ::"v"(pc[wq]), "v"(rs));
      };
      const float shift = kPShiftLog2 - m;
      // PV(j-1) with the first four code words, then S(j+1) with the last four. The V and K
      // operands were read above; each MFMA waits only for its own.
      constexpr int WPV = 4 / DB, WS = 4 / NSM;   // code words per PV and per S MFMA
      static_assert(WPV * DB == 4 && WS * NSM == 4, "the code words split evenly over the MFMAs");
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db] = mfma_fp8(vop[db], pop, o[db]);
#pragma unroll
        for (int wq = db * WPV; wq < (db + 1) * WPV; ++wq) codes(wq, shift);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < NSM; ++e) {
        sn[e % KB] = mfma_fp8(kop[e], qop[e / KB], sn[e % KB]);
#pragma unroll
        for (int wq = 4 + e * WS; wq < 4 + (e + 1) * WS; ++wq) codes(wq, shift);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // a term can exceed 448 only if its lane's sum does (the first tile with an admitted key
      // always does: m starts at -1e30). Then the row max decides whether m moves; O already
      // holds PV(j-1), whose codes were taken against the old m, and is rescaled with l.
      if (__builtin_amdgcn_ballot_w64(!(rs <= kSumBound8))) {
        float mx = sc[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        const float mxc = pair_max(mx) * c2;
        const float m_new = mxc > m + kTau8 ? mxc + kLift : m;
        if (__builtin_amdgcn_ballot_w64(m_new != m)) {
          const float alpha = __builtin_amdgcn_exp2f(m - m_new);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
          m = m_new;
          rs = -0.f;
#pragma unroll
          for (int wq = 0; wq < 8; ++wq) codes(wq, kPShiftLog2 - m);
        }
      }
      l += rs;
    }
    barrier_keep(CH * ((int)k3 + (int)v1));
    const uint32_t rt = r0;
    r0 = r1;
    r1 = r2;
    r2 = rt;
    k_soff = __builtin_amdgcn_readfirstlane(k_soff + BN * k_rowb);
    v_soff = __builtin_amdgcn_readfirstlane(v_soff + BN * v_rowb);
  };

  // steps tb .. te; the last one only drains PV(te-1)
  for (int t = tb;; t += 2) {
    step(t, sa, sb, pb, pa);
    if (t + 1 > te) break;
    step(t + 1, sb, sa, pa, pb);
    if (t + 2 > te) break;
  }

  // epilogue: O * dv / l (both carry the 2^8 shift), lse = (m + log2(l / 2^8)) * ln 2
  if (!wave_live) return;
  // O (bf16) leaves through LDS as in the fp16/bf16 kernel: each wave writes its 32 rows into a
  // private region of the idle rings in the MFMA layout and stores them back by whole rows
  // (16-byte chunk c of row r at c ^ (r % OCPR)); rows past the sequence are dropped by the
  // buffer range check.
  constexpr int OROWB = D * 2, OCPR = OROWB / 16, RPI = 1024 / OROWB;
  static_assert(WAVES * 32 * OROWB <= 2 * NS * TILEB, "the output stage fits in the rings");
  const uint32_t stage = lds_addr_of(smem) + wave * 32 * OROWB;
  const float l_tot = pair_sum(l);
  const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t w0v = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(o[db][4 * q4 + 0] * inv),
                                                               (__bf16)(o[db][4 * q4 + 1] * inv)});
      const uint32_t w1v = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(o[db][4 * q4 + 2] * inv),
                                                               (__bf16)(o[db][4 * q4 + 3] * inv)});
      lds_write_b64(stage + l32 * OROWB + (((db * 4 + q4) ^ (l32 % OCPR)) << 4) + hl * 8, i32x2{(int)w0v, (int)w1v});
    }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the reads below follow the writes (one wave: in order)
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / OCPR, c = lane % OCPR;
    const i32x4 v = lds_read_b128(stage + r * OROWB + ((c ^ (r % OCPR)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(v, o_r, (uint32_t)(w0 + r) * o_rowb + c * 16, 0, 0);
  }
  if (a.lse != nullptr && hl == 0 && my_row < sv.Nq) {
    const float lse = l_tot > 0.f ? (m - kPShiftLog2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    a.lse[sv.lse0 + my_row] = lse;
  }
}

template <int D>
static hipError_t launch_t(const FwdArgs& a, int64_t grid, hipStream_t stream) {
  constexpr int BN = 64, WAVES = 4;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, BN, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int D, int64_t grid, hipStream_t stream) {
  return D == 64 ? launch_t<64>(a, grid, stream) : launch_t<128>(a, grid, stream);
}

}  // namespace fa
