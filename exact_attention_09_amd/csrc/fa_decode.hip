// fa_decode.hip — attention of a few queries per sequence against a dense or paged key/value
// cache: the decode-shaped workload ("Flash Attention - Fast Memory-Efficient Attention", skill
// page, section "Advanced features": paged KV cache; "FlashAttention V3 principles and practice",
// section 4: KV-cache blocks stored as pages for inference).
//
// Few queries give little parallelism across rows, so the keys are split: one wave per
// (batch, K/V head, block of 32 query rows, key split). The rows of a block are the query heads
// sharing the K/V head times the queries (row r = query head r / Nq of the group, query r % Nq),
// so under MQA/GQA one pass over the cache serves all of them. Per 32-key block the wave loads
// K and V rows with 64-bit per-lane addresses (each key may sit in another page), computes
// S^T = K Q^T with K as the A operand straight from registers, runs the online softmax in its
// registers (one query row per lane pair), and adds V^T P^T with V^T read transposed from its
// own LDS tile. The next two blocks' K and V are in flight during the current one. Each split writes
// its normalised output and lse; fa_decode_merge_kernel combines the splits (or, with one split,
// the wave writes the result itself).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_f16_common.hpp"
#include "fa_kernels.hpp"
#include "fa_mask.hpp"
#include "fa_tile.hpp"

namespace fa {

// Keys a sequence may use: its seqlens_k entry clamped to what the cache can hold.
__device__ inline int dec_len(const DecArgs& a, int b) {
  int cap = a.max_seqlen_k;
  if (a.block_table != nullptr) {
    const int64_t pages = (int64_t)a.max_pages * a.page_size;
    cap = pages < cap ? (int)pages : cap;
  }
  const int n = a.seqlens_k[b];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

template <class TR, int D, bool PAGED>
__global__ void __launch_bounds__(64) fa_decode_kernel(DecArgs a) {
  using T = OpTile<D>;
  constexpr int ES = 2, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char vtile[32 * T::ROWB];   // the wave's 32 V rows
  // the wave's 32 query rows can be read back from LDS for every block instead of kept in
  // registers (measured no faster: off)
  constexpr bool Q_IN_LDS = false;
  __shared__ __attribute__((aligned(16))) char qtile[Q_IN_LDS ? 32 * T::ROWB : 16];
  extern __shared__ int ptab[];   // paged cache: the page ids of this split (pages_per_split)

  // register buffers: blocks in flight two ahead of their use (at D = 128 this takes the kernel
  // past 256 registers, to one wave per SIMD; one buffer fewer measured slower all the same)
  constexpr int NB = 3;
  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  // Which (pair, split): pair = (b * Hkv + hk) * row_blocks + rb. Workgroups are dealt
  // round-robin to the 8 XCDs. With few splits per pair, consecutive ids take the same split of
  // consecutive pairs (split-major): split-fastest ids would put split s on the XCDs congruent to
  // s, and the first splits are the fullest. With many splits, the splits of a pair are
  // consecutive (each XCD then meets every split index).
  const int pairs = a.B * a.Hkv * a.row_blocks;
  int s, u;
  if (a.n_split < 16) {
    s = (int)blockIdx.x / pairs;
    u = (int)blockIdx.x - s * pairs;
  } else {
    s = (int)blockIdx.x % a.n_split;
    u = (int)blockIdx.x / a.n_split;
  }
  const int rb = u % a.row_blocks;
  u /= a.row_blocks;
  const int hk = u % a.Hkv, b = u / a.Hkv;

  const int len = dec_len(a, b);
  const int k_begin = s * a.split_keys;
  const int k_end = min(len, k_begin + a.split_keys);
  if (k_begin >= k_end && a.n_split > 1) return;   // the merge reads only splits that hold keys

  // this lane's query row
  const int rows = a.group * a.Nq;
  const int r = rb * 32 + l32;
  const bool row_ok = r < rows;
  const int qi = row_ok ? r % a.Nq : 0;
  const int h = hk * a.group + (row_ok ? r / a.Nq : 0);
  const MaskSpec ms{a.Nq, len, a.causal, a.wl, a.wr};
  const int64_t lo_i = key_lo(ms, qi), hi_i = key_hi(ms, qi);
  // keys some query admits, and keys every query admits (both bounds grow with the query)
  const int64_t any_lo = key_lo(ms, 0), any_hi = key_hi(ms, a.Nq - 1);
  const int64_t all_lo = key_lo(ms, a.Nq - 1), all_hi = key_hi(ms, 0);
  const int jb = (int)max((int64_t)k_begin, any_lo) & ~31;
  const int je = (int)min((int64_t)k_end, any_hi + 1);

  i32x4 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = i32x4{};
    if (row_ok)
      qop[ks] = *(const i32x4*)((const char*)a.q + (b * a.q_b + qi * a.q_n + h * a.q_h + ks * 16 + hl * 8) * ES);
  }
  const uint32_t qt = lds_addr_of(qtile);
  if constexpr (Q_IN_LDS) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *(__attribute__((address_space(3))) i32x4*)(uintptr_t)(qt + T::row_off(l32, ks, hl)) = qop[ks];
  }

  // Blocks of 32 keys jb, jb + 32, ... below je. Lane l32 loads key j0 + l32 of a block (clamped
  // to the split's last key: keys past it are masked, and their V rows are real, finite cache rows,
  // so p = 0 meets a finite V). A block's K and V go to one of NB register buffers, NB - 1 blocks
  // ahead of its use. Loads run unconditionally (blocks past the last one reload it): with no
  // branch around them the compiler's wait counts stay exact. With a paged cache the split's page
  // ids are first copied to LDS (one HBM round trip per split instead of one per block).
  const int nblk = jb < je ? (je - jb + 31) / 32 : 0;
  auto key_of = [&](int m) { return min(jb + min(m, nblk - 1) * 32 + l32, k_end - 1); };
  const int first_page = PAGED && nblk > 0 ? k_begin / a.page_size : 0;
  if constexpr (PAGED) {
    if (nblk > 0) {
      const int* table_row = a.block_table + (int64_t)b * a.max_pages;
      const int ne = (k_end - 1) / a.page_size - first_page + 1;   // <= pages_per_split
      for (int e = lane; e < ne; e += 64) {
        const int pg = table_row[first_page + e];
        ptab[e] = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      }
    }
  }
  auto load_block = [&](int m, i32x4 (&kr)[KS], i32x4 (&vr)[KS]) {
    const int j = key_of(m);
    int64_t krow, vrow;
    if constexpr (PAGED) {
      const int pg = ptab[j / a.page_size - first_page];
      const int slot = j % a.page_size;
      krow = pg * a.k_b + (int64_t)slot * a.k_n;
      vrow = pg * a.v_b + (int64_t)slot * a.v_n;
    } else {
      krow = b * a.k_b + (int64_t)j * a.k_n;
      vrow = b * a.v_b + (int64_t)j * a.v_n;
    }
    const char* ka = (const char*)a.kc + (krow + hk * a.k_h + hl * 8) * ES;
    const char* va = (const char*)a.vc + (vrow + hk * a.v_h + hl * 8) * ES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[ks] = *(const i32x4*)(ka + ks * 16 * ES);
      vr[ks] = *(const i32x4*)(va + ks * 16 * ES);
    }
  };

  const uint32_t vt = lds_addr_of(vtile);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e8 = 0; e8 < 2; ++e8) toff[db][e8] = T::tr_off(lane, db, e8);
  uint32_t vbase[DB][2];
  tr_bases<D>(vt, toff, vbase);

  const float c2 = a.scale_log2;
  float m = -1e30f, l = 0.f;   // running max (base 2, finite start: a fully masked block gives p = 0)
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  // block n: issue the loads of block n + NB - 1 (into `nk`, `nv`), then compute block n from
  // `ck`, `cv`
  auto step = [&](int n, const i32x4 (&ck)[KS], const i32x4 (&cv)[KS], i32x4 (&nk)[KS], i32x4 (&nv)[KS]) {
    load_block(n + NB - 1, nk, nv);
    const int j0 = jb + n * 32;
    // V(j0) into the wave's tile (row l32, chunk 2 ks + hl); the wave's own transpose reads below
    // are ordered after these writes by the LDS queue
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *(__attribute__((address_space(3))) i32x4*)(uintptr_t)(vt + T::row_off(l32, ks, hl)) = cv[ks];
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4 qk = qop[ks];
      if constexpr (Q_IN_LDS) qk = lds_read_b128(qt + T::row_off(l32, ks, hl));
      sc = TR::mfma(ck[ks], qk, sc);
    }
    // accumulator e: key j0 + (e/4)*8 + hl*4 + e%4 for this lane's row
    const bool full = j0 >= all_lo && j0 + 31 <= all_hi && j0 + 31 < k_end;
    if (!full) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + (e >> 2) * 8 + hl * 4 + (e & 3);
        const bool ok = row_ok && j < k_end && j >= lo_i && j <= hi_i;
        sc[e] = ok ? sc[e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = pair_max(mx) * c2;
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    uint32_t pk[8];
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], c2, -m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e + 1], c2, -m));
      pk[e >> 1] = TR::pack(p0, p1);
      rs = TR::sum2(rs, pk[e >> 1], p0, p1);
    }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    // O^T += V^T P^T (k = the block's 32 keys, two halves of 16)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const i32x4 pop = i32x4{(int)pk[4 * half], (int)pk[4 * half + 1], (int)pk[4 * half + 2], (int)pk[4 * half + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = TR::mfma(tr_operand<D>(vbase, 0, half, db), pop, o[db]);
    }
  };

  // NB register buffers per trip, each in a fixed role: no register copies between blocks. The
  // loop runs whole trips of NB blocks and the last blocks after it: with no exit from the middle
  // of a trip (and no path into the loop that skips the first loads), the back edge is the only
  // way back to the top, and the compiler's wait counts keep NB - 1 blocks in flight (an exit in
  // mid-trip made it wait for every load at the top of each trip).
  i32x4 k0[KS], v0[KS], k1[KS], v1[KS], k2[KS], v2[KS];
  if (nblk > 0) {
    load_block(0, k0, v0);
    if constexpr (NB == 3) {
      load_block(1, k1, v1);
      int n = 0;
      for (; n + 3 <= nblk; n += 3) {
        step(n, k0, v0, k2, v2);
        step(n + 1, k1, v1, k0, v0);
        step(n + 2, k2, v2, k1, v1);
      }
      if (n < nblk) {
        step(n, k0, v0, k2, v2);
        if (n + 1 < nblk) step(n + 1, k1, v1, k0, v0);
      }
    } else {
      int n = 0;
      for (; n + 2 <= nblk; n += 2) {
        step(n, k0, v0, k1, v1);
        step(n + 1, k1, v1, k0, v0);
      }
      if (n < nblk) step(n, k0, v0, k1, v1);
    }
  }

  if (!row_ok) return;
  const float l_tot = pair_sum(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  const int64_t row_id = ((int64_t)b * a.Hq + h) * a.Nq + qi;
  if (a.n_split == 1) {
    char* orow = (char*)a.o + (b * a.o_b + qi * a.o_n + h * a.o_h) * ES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w0 = TR::pack(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv);
        const uint32_t w1 = TR::pack(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
        *(i32x2*)(orow + (db * 32 + q4 * 8 + hl * 4) * ES) = i32x2{(int)w0, (int)w1};
      }
    if (a.lse != nullptr && hl == 0) a.lse[row_id] = lse;
    return;
  }
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Nq;
  float* prow = a.part + ((int64_t)s * nrows + row_id) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *(f32x4*)(prow + db * 32 + q4 * 8 + hl * 4) =
          f32x4{o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv};
  if (hl == 0) a.part[(int64_t)a.n_split * nrows * D + (int64_t)s * nrows + row_id] = lse;
}

// out = sum over the splits s that hold keys of exp(lse_s - lse) * out_s, lse = log sum exp(lse_s):
// 8 columns of one query row per thread.
template <class TR, int D>
__global__ void __launch_bounds__(256) fa_decode_merge_kernel(DecArgs a) {
  constexpr int ES = 2;
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Nq;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row_id = gid / (D / 8);
  if (row_id >= nrows) return;
  const int col = (int)(gid - row_id * (D / 8)) * 8;
  const int qi = (int)(row_id % a.Nq);
  const int64_t bh = row_id / a.Nq;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int len = dec_len(a, b);
  const int ns = (len + a.split_keys - 1) / a.split_keys;
  const float* plse = a.part + (int64_t)a.n_split * nrows * D;
  constexpr float kLog2e = 1.44269504088896340736f;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, plse[(int64_t)s * nrows + row_id]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx > -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < ns; ++s) sum += __builtin_amdgcn_exp2f((plse[(int64_t)s * nrows + row_id] - mx) * kLog2e);
    lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
    for (int s = 0; s < ns; ++s) {
      const float w = __builtin_amdgcn_exp2f((plse[(int64_t)s * nrows + row_id] - lse) * kLog2e);
      const float* src = a.part + ((int64_t)s * nrows + row_id) * D + col;
      const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * x0[e];
        acc[4 + e] += w * x1[e];
      }
    }
  }
  const i32x4 packed = i32x4{(int)TR::pack(acc[0], acc[1]), (int)TR::pack(acc[2], acc[3]), (int)TR::pack(acc[4], acc[5]),
                             (int)TR::pack(acc[6], acc[7])};
  *(i32x4*)((char*)a.o + (b * a.o_b + qi * a.o_n + h * a.o_h + col) * ES) = packed;
  if (a.lse != nullptr && col == 0) a.lse[row_id] = lse;
}

template <class TR, int D>
static hipError_t launch_decode_t(const DecArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * a.Hkv * a.row_blocks * a.n_split;
  if (a.block_table != nullptr)
    hipLaunchKernelGGL((fa_decode_kernel<TR, D, true>), dim3((unsigned)units), dim3(64),
                       (size_t)a.pages_per_split * 4, stream, a);
  else
    hipLaunchKernelGGL((fa_decode_kernel<TR, D, false>), dim3((unsigned)units), dim3(64), 0, stream, a);
  if (a.n_split > 1) {
    const int64_t threads = (int64_t)a.B * a.Hq * a.Nq * (D / 8);
    hipLaunchKernelGGL((fa_decode_merge_kernel<TR, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_decode_t<F16, 64>(a, stream) : launch_decode_t<F16, 128>(a, stream);
  return D == 64 ? launch_decode_t<BF16, 64>(a, stream) : launch_decode_t<BF16, 128>(a, stream);
}

}  // namespace fa
