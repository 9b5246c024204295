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
//  * One workgroup per (batch, query head, tile of BM = 32 * QB * WAVES query rows); each 64-lane
//    wave owns QB consecutive blocks of 32 query rows. With QB = 2 (head dimension 64) every K
//    and V operand a wave reads from LDS serves both of its blocks, which halves the LDS reads
//    and the HBM -> LDS bytes per product. The grid is remapped so that the workgroups one XCD
//    receives (hardware deals blocks round-robin over the 8 XCDs) cover whole heads: a head's K/V
//    stays in that XCD's L2. Under a causal mask a head's heaviest query tiles start first.
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
//    (no register staging), into three-slot rings: step j issues the loads of K(j+3) and V(j+1),
//    first read in step j+2, so each load has two steps to land. Each lane's 16 bytes land at its
//    own slot position; which global chunk a lane fetches implements the LDS swizzle.
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

template <class TR, int D, int BN, int WAVES, int QB, bool SP, int HP>
__global__ void __launch_bounds__(WAVES * 64) fa_fwd_kernel(FwdArgs a) {
  constexpr int NT = WAVES * 64;        // threads per workgroup
  constexpr int WR = 32 * QB;           // query rows per wave: QB blocks of 32
  constexpr int WPH = WAVES / HP;       // waves per query head: HP heads sharing a K/V head
  constexpr int BM = WPH * WR;          // query rows per workgroup (of each of its HP heads)
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
  static_assert(!SP || QB == 1, "block-sparse launches keep one query block per wave");
  static_assert(WAVES % HP == 0 && (!SP || HP == 1), "whole waves per head; block-sparse keeps one head");

  constexpr int NS = 3;                 // ring slots per tensor
  __shared__ __attribute__((aligned(16))) char smem[2 * NS * TILEB];  // [K slots | V slots]
  char* const kring = smem;
  char* const vring = smem + NS * TILEB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;      // half of the wave: which 16 of a block's 32 keys / k-slots
  const int l32 = lane & 31;     // query column of this lane inside each 32-row block of the wave

  // ---- which (batch, head, query tile) this workgroup computes. With HP > 1 the launch order
  // counts groups of HP consecutive query heads (they share a K/V head: HP divides the GQA group),
  // and wave w serves head HP * group + w / WPH: every K/V tile brought into LDS serves HP heads.
  int b, hs, qt;
  schedule_block(blockIdx.x, a.sched, &b, &hs, &qt);
  const int h = hs * HP + wave / WPH;
  const int hk = (int)fdiv((uint32_t)hs, a.sched.group);   // MQA/GQA: K/V head of this query head
  const int q0 = qt * BM;
  const SeqView sv = seq_view(a, b, h, D, ES, ES);
  if (q0 >= sv.Nq) return;                       // past the end of a shorter packed sequence

  const MaskSpec ms{sv.Nq, sv.Nk, a.causal, a.wl, a.wr};

  const char* qb = (const char*)a.q + (sv.q0 + h * a.q_h) * ES;
  const char* kbp = (const char*)a.k + (sv.k0 + hk * a.k_h) * ES;
  const char* vbp = (const char*)a.v + (sv.v0 + hk * a.v_h) * ES;
  char* ob = (char*)a.o + (sv.o0 + h * a.o_h) * ES;
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc(qb, sv.q_bytes);
  const __amdgpu_buffer_rsrc_t o_r = make_rsrc(ob, sv.o_bytes);
  const uint32_t q_rowb = (uint32_t)(a.q_n * ES), k_rowb = (uint32_t)(a.k_n * ES);
  const uint32_t v_rowb = (uint32_t)(a.v_n * ES), o_rowb = (uint32_t)(a.o_n * ES);

  // ---- K/V tiles this workgroup visits, and this wave's rows (QB consecutive blocks of 32)
  const int wg_last = min(q0 + BM, sv.Nq) - 1;
  int tb, te;
  tile_range(ms, q0, wg_last, BN, &tb, &te);
  const int w0 = q0 + (wave % WPH) * WR;
  const bool wave_live = w0 < sv.Nq;
  const int w1 = min(w0 + WR - 1, sv.Nq - 1);
  int my_row[QB];   // this lane's query row in each block
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) my_row[qb2] = w0 + qb2 * 32 + l32;

  // ---- block-sparse: the tiles of [tb, te) that the block mask sets for one of the workgroup's
  // mask rows, compacted into LDS by wave 0 (sp_list: tile ids, then a bit per mask row, then the
  // count). Steps then run over positions 0 .. n of this list instead of tiles tb .. te, and a
  // tile whose bit is clear for a wave's own mask row is masked entirely for that wave.
  extern __shared__ int sp_list[];
  int sp_n = 0, sp_row = 0;
  if constexpr (SP) {
    const int mr0 = q0 / kSparseBlockQ;
    const int nrows = min(BM / kSparseBlockQ, a.nqb - mr0);
    sp_row = w0 / kSparseBlockQ - mr0;
    const uint8_t* mrow = a.block_mask + ((int64_t)(a.mask_heads == 1 ? 0 : h) * a.nqb + mr0) * a.nkb;
    if (wave == 0) {
      int cnt = 0;
      for (int base = tb; base < te; base += 64) {
        const int t = base + lane;
        int bits = 0;
        if (t < te)
          for (int r = 0; r < nrows; ++r) bits |= (mrow[(int64_t)r * a.nkb + t] != 0) << r;
        const uint64_t set = __builtin_amdgcn_ballot_w64(bits != 0);
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(set >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)set, 0));
        if (bits != 0) {
          sp_list[pos] = t;
          sp_list[a.nkb + pos] = bits;
        }
        cnt += __builtin_popcountll(set);
      }
      if (lane == 0) sp_list[2 * a.nkb] = cnt;
    }
    __syncthreads();
    sp_n = __builtin_amdgcn_readfirstlane(sp_list[2 * a.nkb]);
  }
  // tile of step position p (SP) and whether this wave's mask row admits it; positions past the
  // list map to a tile past every key, which the element masks clear entirely
  auto sp_tile = [&](int p) {
    const int t = __builtin_amdgcn_readfirstlane(sp_list[p < sp_n ? p : 0]);   // index kept in range
    return p < sp_n ? t : te + 2;
  };
  auto sp_admits = [&](int p) {
    const int bits = __builtin_amdgcn_readfirstlane(sp_list[a.nkb + (p < sp_n ? p : 0)]);
    return p < sp_n && ((bits >> sp_row) & 1);
  };
  const int pb0 = SP ? 0 : tb, pe = SP ? sp_n : te;   // step positions pb0 .. pe

  // Q operands (B operand of S^T): block qb2's row, head-dim slots ks*16 + hl*8 .. +7; loaded in
  // the prologue, behind the first K/V tile loads
  i32x4 qop[QB][KS];

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
  const BufDesc k_d = make_desc(kbp, sv.k_bytes), v_d = make_desc(vbp, sv.v_bytes);
  const uint32_t kring_a = lds_addr_of(kring), vring_a = lds_addr_of(vring);
  // The CH loads of one tile: soff is the tile's byte offset in the head, lds its ring slot.
  auto dma = [&](const BufDesc& d, const uint32_t* goff, uint32_t soff, uint32_t lds) {
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(d, goff[i], soff, lds + wave * 64 * 16 + i * NT * 16);
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

  // ---- prologue loads, issued before the rest of the set-up so that their latency overlaps it:
  // K(tb), K(tb+1), V(tb), K(tb+2) (positions 0, 1, 2 of the tile list when block-sparse) into
  // ring slots 0, 1, 0, 2, and this wave's Q rows
  if (pb0 < pe) {
    const int t0 = SP ? sp_tile(0) : tb, t1 = SP ? sp_tile(1) : tb + 1, t2 = SP ? sp_tile(2) : tb + 2;
    dma(k_d, kgoff, (uint32_t)(t0 * BN) * k_rowb, kring_a);
    if (pb0 + 1 < pe) dma(k_d, kgoff, (uint32_t)(t1 * BN) * k_rowb, kring_a + TILEB);
    dma(v_d, vgoff, (uint32_t)(t0 * BN) * v_rowb, vring_a);
    if (pb0 + 2 < pe) dma(k_d, kgoff, (uint32_t)(t2 * BN) * k_rowb, kring_a + 2 * TILEB);
  }
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[qb2][ks] = __builtin_amdgcn_raw_buffer_load_b128(q_r, (uint32_t)my_row[qb2] * q_rowb + (ks * 16 + hl * 8) * ES,
                                                           0, 0);

  // Key bounds of the wave's first and last rows, clamped to [-1, Nk] (wave-uniform scalars).
  // Each row admits an interval of keys and both ends grow with the row, so the tiles holding
  // an admitted key for some row of the wave form an interval [jlo, jhi), and the tiles admitted
  // for every row another one, [flo, fhi), inside it.
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
  // the keys this lane's row in each block admits: [lo_i, lo_i + span_i)
  int lo_i[QB];
  uint32_t span_i[QB];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    lo_i[qb2] = clamp_key(key_lo(ms, my_row[qb2]));
    const int hi_i = clamp_key(key_hi(ms, my_row[qb2]));
    span_i[qb2] = hi_i >= lo_i[qb2] ? (uint32_t)(hi_i - lo_i[qb2] + 1) : 0u;
  }

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

  const float c2 = a.scale_log2;
  // Reference max of score * c2 for this lane's query in each block. It starts at a huge negative
  // finite value rather than -inf: the first tile with an admitted key then overflows the sum
  // bound and sets the reference (see kSumBound), while a fully masked tile still gives
  // p = exp2(-inf) = 0.
  constexpr float kRefStart = -1e30f;
  float m[QB], l[QB];    // l: this lane's share of the running sum (lanes l, l^32 split the keys)
  f32x16 o[QB][DB];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    m[qb2] = kRefStart;
    l[qb2] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb2][db] = f32x16{};
  }

  // ---- building blocks of one step
  // Products of a tile, numbered in issue order. S MFMA i: K operand i / QB (k-step (i/QB) / KB,
  // key block (i/QB) % KB) against query block i % QB, so each K operand read from LDS serves the
  // QB blocks back to back; accumulators that depend on each other are KB * QB products apart.
  // PV MFMA i: V operand i / QB (key block, half, column block), query block i % QB.
  auto mfma_s = [&](const i32x4& kop, f32x16 (&s)[QB][KB], int i) {
    const int u = i / QB, qb2 = i % QB;
    s[qb2][u % KB] = TR::mfma(kop, qop[qb2][u / KB], s[qb2][u % KB]);
  };
  auto mfma_pv = [&](const i32x4& vop, const uint32_t (&pk)[QB][KB][8], int i) {
    const int u = i / QB, qb2 = i % QB;
    const int kb = u / (2 * DB), half = (u / DB) % 2, db = u % DB;
    const i32x4 pop = i32x4{(int)pk[qb2][kb][4 * half + 0], (int)pk[qb2][kb][4 * half + 1],
                            (int)pk[qb2][kb][4 * half + 2], (int)pk[qb2][kb][4 * half + 3]};
    o[qb2][db] = TR::mfma(vop, pop, o[qb2][db]);
  };
  // Softmax of score pair number i of query block qb2 (key block i / 8, accumulator entries
  // 2 (i % 8) and + 1): p = exp2(s * c - mref), packed to the MFMA type, added to the row sum.
  auto p_pair = [&](const f32x16 (&sc)[KB], uint32_t (&pk)[KB][8], float& rs, float mref, int i) {
    const int kb = i / 8, r = (i % 8) * 2;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c2, -mref));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r + 1], c2, -mref));
    pk[kb][r >> 1] = TR::pack(p0, p1);
    rs = TR::sum2(rs, pk[kb][r >> 1], p0, p1);
  };
  constexpr int NK = KS * KB;           // K operands per tile
  constexpr int NV = KB * 2 * DB;       // V operands per tile
  constexpr int NSM = NK * QB;          // S MFMAs per tile
  constexpr int NPV = NV * QB;          // PV MFMAs per tile
  constexpr int NPB = KB * 8;           // score pairs per lane per tile and query block
  constexpr int NPAIR = NPB * QB;
  static_assert(NSM == NPV && (2 * NSM) % NPAIR == 0, "the interleave pairs S and PV MFMAs one to one");
  auto softmax_all = [&](f32x16 (&sc)[KB], uint32_t (&pk)[KB][8], float& rs, float mref) {
    rs = 0.f;
#pragma unroll
    for (int i = 0; i < NPB; ++i) p_pair(sc, pk, rs, mref, i);
  };
  // Rebase when a p may exceed the bound (see kSumBound): m moves to the running max, O and l
  // are rescaled, p is recomputed. O must already hold every PV product issued against the old m.
  auto check_rebase = [&](f32x16 (&sc)[KB], uint32_t (&pk)[KB][8], float& rs, int qb2) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumBound))) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      const float m_new = fmaxf(m[qb2], pair_max(mx) * c2);   // finite: m starts finite
      const float alpha = __builtin_amdgcn_exp2f(m[qb2] - m_new);
      l[qb2] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb2][db] *= alpha;
      m[qb2] = m_new;
      softmax_all(sc, pk, rs, m[qb2]);
    }
    l[qb2] += rs;
  };
  auto mask_tile = [&](f32x16 (&sc)[QB][KB], int t) {
    // key of accumulator r in block kb is t*BN + kb*32 + (r/4)*8 + hl*4 + r%4
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      const int jl = t * BN + hl * 4 - lo_i[qb2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jl + kb * 32 + (r >> 2) * 8 + (r & 3);
          sc[qb2][kb][r] = (uint32_t)j < span_i[qb2] ? sc[qb2][kb][r] : -INFINITY;
        }
    }
  };

  // ---- software pipeline. Step j: loads of K(j+3) and V(j+1) are issued; then PV(j-1) and
  // S(j+1) run on the matrix pipe while the softmax of tile j (scores computed in step j-1) runs
  // on the vector pipe. PV lags one tile so that its operand P(j-1) is ready at the start of the
  // step. The three products of a step are independent and are issued as one interleaved
  // sequence: each MFMA is followed by the softmax of a share of the tile's scores, so a single
  // wave keeps both pipes busy.
  // A wave runs this sequence in every step from jlo - 1 to jhi (the tiles it needs, plus one on
  // each side for the lagging PV and the leading S) and skips the others; tiles outside its
  // interval are masked like partial ones, so their P is exactly zero and their PV adds nothing.
  // Tile j of either tensor sits in ring slot (j - tb) % 3; a slot is refilled one step after
  // its last read, behind the step's closing barrier. r0, r1, r2 are the byte offsets of slots
  // (j - tb) % 3, (j - tb + 1) % 3 and (j - tb + 2) % 3.
  const int need_lo = jlo - 1;
  const uint32_t need_n = jlo < jhi ? (uint32_t)(jhi - jlo + 2) : 0u;
  const uint32_t full_n = fhi > flo ? (uint32_t)(fhi - flo) : 0u;

  uint32_t r0 = 0, r1 = TILEB, r2 = 2 * TILEB;
  uint32_t k_soff = (uint32_t)((tb + 3) * BN) * k_rowb;   // byte offset of K(j+3)
  uint32_t v_soff = (uint32_t)((tb + 1) * BN) * v_rowb;   // byte offset of V(j+1)
  // V slot 2 stands for V(tb-1), read (against P = 0) by the first step before any load fills
  // it: zero it so that the product is exactly zero.
#pragma unroll
  for (int c = tid * 16; c < TILEB; c += NT * 16) *(i32x4*)(vring + 2 * TILEB + c) = i32x4{};
  // Q (and with it the first tiles) must have landed before the pipelined loop: without this
  // wait the compiler's wait-count analysis, merging the loop back edge, would make every
  // iteration wait on the prefetches.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  barrier_keep(0);
  f32x16 sa[QB][KB], sb[QB][KB];
  uint32_t pa[QB][KB][8], pb[QB][KB][8];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 8; ++r) pa[qb2][kb][r] = pb[qb2][kb][r] = 0u;
  {
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sa[qb2][kb] = f32x16{};
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const i32x4 kop = lds_read_b128(opaque_vbase(kring_a + koff[u / KB]) + (u % KB) * 32 * ROWB);
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) mfma_s(kop, sa, u * QB + qb2);
    }
  }
  barrier_keep(0);   // every wave has read K(tb) before step tb refills its slot

  auto step = [&](int j, f32x16 (&sc)[QB][KB], f32x16 (&sn)[QB][KB], const uint32_t (&pp)[QB][KB][8],
                  uint32_t (&pc)[QB][KB][8]) {
    const bool k3 = j + 3 < pe, v1 = j + 1 < pe;
    if (k3) dma(k_d, kgoff, SP ? (uint32_t)(sp_tile(j + 3) * BN) * k_rowb : k_soff, kring_a + r0);
    if (v1) dma(v_d, vgoff, SP ? (uint32_t)(sp_tile(j + 1) * BN) * v_rowb : v_soff, vring_a + r1);
    if (SP || (uint32_t)(j - need_lo) < need_n) {
      if constexpr (SP) {
        const int tj = sp_tile(j);
        if (!sp_admits(j)) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) sc[0][kb] = f32x16{} - INFINITY;
        } else if (!((uint32_t)(tj - flo) < full_n)) {
          mask_tile(sc, tj);
        }
      } else {
        if (!((uint32_t)(j - flo) < full_n)) mask_tile(sc, j);
      }
      // A row's first tile with an admitted key would trip the sum bound (its reference is still
      // the start value) and pay a second softmax pass in check_rebase; the row's reference is
      // set from this tile's max instead. Nothing has been accumulated for such a row (l = 0,
      // O = 0), so no rescale is due; a row whose keys in this tile are all masked keeps the
      // start value. A row's first admitted key grows with the row, so over the wave's 32 * QB
      // rows it spans at most 32 * QB keys: QB + 1 tiles from the wave's first. Only those steps
      // look; a row first admitted later (the check is an optimisation) goes through
      // check_rebase as before.
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) {
        if ((SP || (uint32_t)(j - jlo) <= (uint32_t)QB) && __builtin_amdgcn_ballot_w64(m[qb2] == kRefStart)) {
          float mx = sc[qb2][0][0];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qb2][kb][r]);
          const float mt = pair_max(mx) * c2;
          if (m[qb2] == kRefStart) m[qb2] = fmaxf(kRefStart, mt);
        }
      }
      // Operand u of the step (even u: K operand u / 2, read by rows from LDS; odd u: V^T
      // operand u / 2, read by transpose reads), read PF operands ahead of its first use. At
      // D = 64 every read is issued up front (registers allow it and it measured fastest) and
      // each MFMA waits only for its own operand (the compiler's per-use waits); at D = 128 a
      // short distance keeps the kernel within 256 registers, so two waves share each SIMD.
      const uint32_t kslot = kring_a + r1, vslot = vring_a + r2;   // K(j+1), V(j-1)
      uint32_t kbase[KS], vbase[DB];
#pragma unroll
      for (int k = 0; k < KS; ++k) kbase[k] = opaque_vbase(kslot + koff[k]);
#pragma unroll
      for (int db = 0; db < DB; ++db) vbase[db] = opaque_vbase(vslot + voff[db]);
      constexpr int NOP = NK + NV, NM = NSM + NPV, PF = D == 64 ? NOP : 3;
      i32x4 opnd[NOP];
      auto read_operand = [&](int u) {
        const int idx = u / 2;
        if (u % 2 == 0) {
          opnd[u] = lds_read_b128(kbase[idx / KB] + (idx % KB) * 32 * ROWB);
        } else {
          const int kb = idx / (2 * DB), half = (idx / DB) % 2, db = idx % DB;
          const uint32_t p = vbase[db] + (kb * 32 + half * 16) * ROWB;
          const i32x2 v0 = lds_read_tr16(p), v1 = lds_read_tr16(p + 8 * ROWB);
          opnd[u] = i32x4{v0[0], v0[1], v1[0], v1[1]};
        }
      };
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sn[qb2][kb] = f32x16{};
      float rs[QB];
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) rs[qb2] = 0.f;
#pragma unroll
      for (int u = 0; u < PF; ++u) read_operand(u);
      // The sequence runs at raised issue priority: when both waves of a SIMD are ready, the one
      // inside its sequence (which feeds both pipes) issues first.
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int PER = NM / NPAIR;   // MFMAs per score pair
#pragma unroll
      for (int e = 0; e < NM; ++e) {
        // MFMA e: S MFMA e / 2 (even e) or PV MFMA e / 2 (odd e); operand u of the step
        const int i = e / 2, u = 2 * (i / QB) + (e % 2);
        if (i % QB == 0 && u + PF < NOP) read_operand(u + PF);
        if (e % 2 == 0) mfma_s(opnd[u], sn, i);
        else mfma_pv(opnd[u], pp, i);
        if (e % PER == PER - 1) {
          const int pi = e / PER, qb2 = pi / NPB, pj = pi % NPB;
          p_pair(sc[qb2], pc[qb2], rs[qb2], m[qb2], pj);
          // keep the pair in this group (the compiler would otherwise gather the softmax)
          asm volatile("" ::"v"(pc[qb2][pj / 8][pj % 8]), "v"(rs[qb2]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) check_rebase(sc[qb2], pc[qb2], rs[qb2], qb2);
    }
    // K(j+2) and V(j) must have landed for the next step; this step's loads stay in flight
    barrier_keep(CH * ((int)k3 + (int)v1));
    const uint32_t rt = r0;
    r0 = r1;
    r1 = r2;
    r2 = rt;
    k_soff = __builtin_amdgcn_readfirstlane(k_soff + BN * k_rowb);
    v_soff = __builtin_amdgcn_readfirstlane(v_soff + BN * v_rowb);
  };

  // Steps tb .. te; the last one only drains PV(te-1). Two steps per trip swap the roles of the
  // S and P arrays; the exits after either step keep the loop-carried values in place.
  for (int t = pb0;; t += 2) {
    step(t, sa, sb, pb, pa);
    if (t + 1 > pe) break;
    step(t + 1, sb, sa, pa, pb);
    if (t + 2 > pe) break;
  }


  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2
  if (!wave_live) return;
  // O leaves through LDS: each wave writes one 32-row block of its output there in the MFMA
  // layout (8 bytes per lane and row) and reads it back by rows, so that each store writes whole
  // rows (64 lanes x 16 bytes) instead of 16 bytes in each of 32 rows. The rings are free: the
  // last step's barrier follows every wave's last LDS read and load. Each wave has its own
  // 32 * ROWB-byte region; 16-byte chunk c of row r sits at chunk c ^ (r % CPR), so neither the
  // column-wise writes nor the row-wise reads meet bank conflicts. Rows past the sequence are
  // written to LDS and then dropped by the buffer range check of their stores.
  static_assert(WAVES * 32 * ROWB <= 2 * NS * TILEB, "the output stage fits in the rings");
  constexpr int RPI = 1024 / ROWB;   // rows one 64-lane, 16-byte access covers
  const uint32_t stage = lds_addr_of(smem) + wave * 32 * ROWB;
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const float l_tot = pair_sum(l[qb2]);
    const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w0v = TR::pack(o[qb2][db][4 * q4 + 0] * inv, o[qb2][db][4 * q4 + 1] * inv);
        const uint32_t w1v = TR::pack(o[qb2][db][4 * q4 + 2] * inv, o[qb2][db][4 * q4 + 3] * inv);
        lds_write_b64(stage + l32 * ROWB + (((db * 4 + q4) ^ (l32 % CPR)) << 4) + hl * 8, i32x2{(int)w0v, (int)w1v});
      }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the reads below follow the writes (one wave: in order)
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CPR, c = lane % CPR;
      const i32x4 v = lds_read_b128(stage + r * ROWB + ((c ^ (r % CPR)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(v, o_r, (uint32_t)(w0 + qb2 * 32 + r) * o_rowb + c * 16, 0, 0);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the next block's writes follow these reads
    if (a.lse != nullptr && hl == 0 && my_row[qb2] < sv.Nq) {
      const float lse = l_tot > 0.f ? (m[qb2] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      a.lse[sv.lse0 + my_row[qb2]] = lse;
    }
  }
}

template <class TR, int D>
static hipError_t launch_t(const FwdArgs& a, int block_n, int qb, int hp, int64_t grid, hipStream_t stream) {
  constexpr int BN = 64, WAVES = D == 64 ? 4 : 8;
  static_assert(BN == kSparseBlockK && (WAVES * 32) % kSparseBlockQ == 0, "tiles nest in the mask's blocks");
  if (a.block_mask != nullptr)
    hipLaunchKernelGGL((fa_fwd_kernel<TR, D, BN, WAVES, 1, true, 1>), dim3((unsigned)grid), dim3(WAVES * 64),
                       (size_t)(2 * a.nkb + 1) * 4, stream, a);
  else if (qb == 2) {   // D = 64: two query blocks per wave, 32-key tiles
    if constexpr (D == 64)
      hipLaunchKernelGGL((fa_fwd_kernel<TR, D, 32, 4, 2, false, 1>), dim3((unsigned)grid), dim3(4 * 64), 0, stream, a);
    else
      return hipErrorInvalidValue;
  } else if (block_n == 32 && hp == 4)   // rows with few keys, 4 query heads of one K/V head
    hipLaunchKernelGGL((fa_fwd_kernel<TR, D, 32, 4, 1, false, 4>), dim3((unsigned)grid), dim3(4 * 64), 0, stream, a);
  else if (block_n == 32)   // rows with few keys: 4 waves, 32-key tiles
    hipLaunchKernelGGL((fa_fwd_kernel<TR, D, 32, 4, 1, false, 1>), dim3((unsigned)grid), dim3(4 * 64), 0, stream, a);
  else if (hp == 4 && WAVES == 8)   // D = 128 with 4-way GQA: 4 heads x 64 rows
    hipLaunchKernelGGL((fa_fwd_kernel<TR, D, BN, WAVES, 1, false, 4>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<TR, D, BN, WAVES, 1, false, 1>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_f16(const FwdArgs& a, int D, int dtype, int block_n, int qb, int hp, int64_t grid,
                          hipStream_t stream) {
  if (dtype == 0)
    return D == 64 ? launch_t<F16, 64>(a, block_n, qb, hp, grid, stream)
                   : launch_t<F16, 128>(a, block_n, qb, hp, grid, stream);
  return D == 64 ? launch_t<BF16, 64>(a, block_n, qb, hp, grid, stream)
                 : launch_t<BF16, 128>(a, block_n, qb, hp, grid, stream);
}

}  // namespace fa
