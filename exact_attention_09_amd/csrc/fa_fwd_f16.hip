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
//  * K and V tiles (BN keys) stream HBM -> LDS with 128-bit buffer loads that write LDS directly
//    (no register staging), into three-slot rings: while tile t is computed, the loads of K(t+3)
//    and V(t+2) are in flight, so each load has two iterations to land. Each lane's 16 bytes land
//    at its own slot position; which global chunk a lane fetches implements the LDS swizzle.
//  * S of tile t+1 is computed while tile t goes through the softmax and the PV product (K runs
//    one tile ahead of V), so the MFMAs of one overlap the VALU work of the other.
//  * Softmax in base 2: t = s * (scale * log2 e); p = exp2(t - m); alpha = exp2(m_old - m_new).
//  * Tiles with no admitted key are skipped; tiles admitted for every pair run without a mask;
//    only partial tiles (the causal diagonal, window edges, the ragged end) are masked.
//  * Ragged sizes: buffer resources bound each head's span, so loads past it return 0 and
//    stores past it are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_f16_common.hpp"
#include "fa_kernels.hpp"
#include "fa_mask.hpp"

namespace fa {

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
  static_assert(ROWB == 128 || ROWB == 256, "swizzles are laid out for 128- or 256-byte rows");

  constexpr int NS = 3;                 // ring slots per tensor
  __shared__ __attribute__((aligned(16))) char smem[2 * NS * TILEB];  // [K0 K1 K2 | V0 V1 V2]
  char* const kring = smem;
  char* const vring = smem + NS * TILEB;

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
  // Key bounds of the wave's first and last rows, clamped to [-1, Nk] (wave-uniform scalars):
  // a tile is skipped if it ends before lo(w0) or starts after hi(w1), and needs no mask if it
  // lies inside [lo(w1), hi(w0)].
  auto clamp_key = [&](int64_t x) { return (int)(x < -1 ? -1 : (x > a.Nk ? a.Nk : x)); };
  const int wlo0 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w0)));
  const int wlo1 = __builtin_amdgcn_readfirstlane(clamp_key(key_lo(ms, w1)));
  const int whi0 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w0)));
  const int whi1 = __builtin_amdgcn_readfirstlane(clamp_key(key_hi(ms, w1)));
  auto tile_live = [&](int t) { return wave_live && t * BN + BN - 1 >= wlo0 && t * BN <= whi1; };
  auto tile_partial = [&](int t) { return !(wlo1 <= t * BN && t * BN + BN - 1 <= whi0); };
  const int my_row = w0 + l32;
  const int lo_i = clamp_key(key_lo(ms, my_row));
  const int hi_i = clamp_key(key_hi(ms, my_row));
  const uint32_t span_i = hi_i >= lo_i ? (uint32_t)(hi_i - lo_i + 1) : 0u;

  // ---- Q operands (B operand of S^T): row my_row, head-dim slots ks*16 + hl*8 .. +7
  i32x4 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qop[ks] = __builtin_amdgcn_raw_buffer_load_b128(q_r, (uint32_t)my_row * q_rowb + (ks * 16 + hl * 8) * ES, 0, 0);
  // Q must have landed before the pipelined loop: without this wait the compiler's wait-count
  // analysis, merging the loop back edge, would make every iteration wait on the prefetches.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  // ---- HBM -> LDS loads of one K or V tile. Load i of a thread writes the 16 bytes at slot
  // position P = (i * NT + tid) * 16; P holds row P / ROWB, physical chunk (P % ROWB) / 16, i.e.
  // logical chunk physical ^ swizzle(row). Rows past the end read as 0 (buffer bounds).
  uint32_t kgoff[CH], vgoff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int pos = (i * NT + tid) * 16, row = pos / ROWB, pc = (pos % ROWB) / 16;
    kgoff[i] = (uint32_t)row * k_rowb + ((pc ^ k_swz<ROWB>(row)) << 4);
    vgoff[i] = (uint32_t)row * v_rowb + ((pc ^ v_swz<ROWB>(row)) << 4);
  }
  const BufDesc k_d = make_desc(kbp, a.k_bytes), v_d = make_desc(vbp, a.v_bytes);
  auto dma = [&](const BufDesc& d, const uint32_t* goff, uint32_t rowb, int t, char* slot) {
    const uint32_t base = (uint32_t)(t * BN) * rowb;
    const uint32_t lds = lds_addr_of(slot) + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(d, goff[i], base, lds + i * NT * 16);
  };
  // Barrier that waits only for this thread's loads older than the newest `pending` ones: a
  // compiler-only fence keeps LDS accesses on their side, and no blanket vmcnt(0) is emitted.
  auto barrier_keep = [&](int pending) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (pending >= 2 * CH) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * CH));   // vmcnt(2CH) lgkmcnt(0)
    else if (pending >= CH) __builtin_amdgcn_s_waitcnt(0x0070 | CH);       // vmcnt(CH)  lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0070);                               // vmcnt(0)   lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // Per-lane LDS offsets. K (A operand of S^T): row kb*32 + l32, chunk 2*ks + hl.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + hl) ^ k_swz<ROWB>(l32)) << 4);
  // V (A operand of O^T, transpose read): within each 16-lane group g, source lane 4t + c reads
  // row 4*(g>>1) + t (+8 for the second read), columns db*32 + (g&1)*16 + 4c .. +3.
  const int g16 = lane >> 4, s16 = lane & 15, tr = s16 >> 2, tc = s16 & 3;
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = db * 4 + (g16 & 1) * 2 + (tc >> 1);
    voff[db] = (4 * (g16 >> 1) + tr) * ROWB + ((chunk ^ v_swz<ROWB>(tr)) << 4) + (tc & 1) * 8;
  }

  auto compute_s = [&](const char* ks, f32x16* s) {
    uint32_t kbase[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) kbase[k] = opaque_vbase(lds_addr_of(ks) + koff[k]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      i32x4 kop[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kop[kb] = lds_read_b128(kbase[k] + kb * 32 * ROWB);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = TR::mfma(kop[kb], qop[k], s[kb]);
    }
  };

  const float c2 = a.scale_log2;
  float m = -INFINITY;   // reference max of score * c2 for this lane's query
  float l = 0.f;         // this lane's share of the running sum (lanes l, l^32 split the keys)
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  // ---- pipeline fill: K(tb), V(tb), K(tb+1) landed; S(tb); V(tb+1), K(tb+2) in flight
  if (tb < te) {
    dma(k_d, kgoff, k_rowb, tb, kring);
    dma(v_d, vgoff, v_rowb, tb, vring);
    if (tb + 1 < te) dma(k_d, kgoff, k_rowb, tb + 1, kring + TILEB);
  }
  barrier_keep(0);
  f32x16 sa[KB], sb[KB];
  if (tb < te && tile_live(tb)) compute_s(kring, sa);
  if (tb + 1 < te) dma(v_d, vgoff, v_rowb, tb + 1, vring + TILEB);
  if (tb + 2 < te) dma(k_d, kgoff, k_rowb, tb + 2, kring + 2 * TILEB);
  barrier_keep(2 * CH);    // K(tb) fully read by every wave before its slot is reused

  // One pipeline step: S(t+1) into sn while tile t (scores in sc) goes through the softmax and
  // the PV product. Two steps per loop trip swap the roles of the two S arrays.
  auto step = [&](int t, f32x16 (&sc)[KB], f32x16 (&sn)[KB]) {
    const int i = t - tb;
    const int s0 = i % NS, s1 = (i + 1) % NS, s2 = (i + 2) % NS;   // ring slots of tiles t, t+1, t+2
    const bool k3 = t + 3 < te, v2 = t + 2 < te;
    // K(t+3) into K(t)'s slot (read last step); V(t+2) into V(t-1)'s slot (read last step)
    if (k3) dma(k_d, kgoff, k_rowb, t + 3, kring + s0 * TILEB);
    if (v2) dma(v_d, vgoff, v_rowb, t + 2, vring + s2 * TILEB);
    if (t + 1 < te && tile_live(t + 1)) compute_s(kring + s1 * TILEB, sn);
    if (tile_live(t)) {
      const int j0 = t * BN;
      // V^T operands for this tile
      i32x4 vop[KB][2][DB];
      {
        const char* vs = vring + s0 * TILEB;
        uint32_t vbase[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) vbase[db] = opaque_vbase(lds_addr_of(vs) + voff[db]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const uint32_t p = vbase[db] + (kb * 32 + half * 16) * ROWB;
              const i32x2 v0 = lds_read_tr16(p), v1r = lds_read_tr16(p + 8 * ROWB);
              vop[kb][half][db] = i32x4{v0[0], v0[1], v1r[0], v1r[1]};
            }
      }
      // mask (partial tiles only): key of accumulator r in block kb is j0 + kb*32 + (r/4)*8 + hl*4 + r%4
      if (tile_partial(t)) {
        const int jl = j0 + hl * 4 - lo_i;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = jl + kb * 32 + (r >> 2) * 8 + (r & 3);
            sc[kb][r] = (uint32_t)j < span_i ? sc[kb][r] : -INFINITY;
          }
      }
      // p = exp2(s * c - m), packed to the MFMA type, and the row sum
      uint32_t pk[KB][8];
      float rs;
      auto exponentiate = [&](float mref) {
        rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c2, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r + 1], c2, -mref));
            pk[kb][r >> 1] = TR::pack(p0, p1);
            rs = TR::sum2(rs, pk[kb][r >> 1], p0, p1);
          }
      };
      exponentiate(m);
      if (__builtin_amdgcn_ballot_w64(!(rs <= kSumBound))) {
        // slow path: move the reference to the running max, rescale, recompute
        float mx = sc[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        const float m_new = fmaxf(m, pair_max(mx) * c2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m = m_new;
        exponentiate(m_use);
      }
      l += rs;
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const i32x4 pop = i32x4{(int)pk[kb][4 * half + 0], (int)pk[kb][4 * half + 1], (int)pk[kb][4 * half + 2],
                                  (int)pk[kb][4 * half + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] = TR::mfma(vop[kb][half][db], pop, o[db]);
        }
    }
    // K(t+2) and V(t+1) must have landed for the next step; this step's loads stay in flight
    barrier_keep(CH * ((int)k3 + (int)v2));
  };

  for (int t = tb; t < te; t += 2) {
    step(t, sa, sb);
    if (t + 1 < te) step(t + 1, sb, sa);
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
