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
// own LDS tile. The next block's K and V are in flight during the current one. Each split writes
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

template <class TR, int D>
__global__ void __launch_bounds__(64) fa_decode_kernel(DecArgs a) {
  using T = OpTile<D>;
  constexpr int ES = 2, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char vtile[32 * T::ROWB];   // the wave's 32 V rows

  const int lane = threadIdx.x, hl = lane >> 5, l32 = lane & 31;
  int u = blockIdx.x;
  const int s = u % a.n_split;
  u /= a.n_split;
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

  // K or V row of key j (a lane's own key): 64-bit address of its first element
  auto row_addr = [&](const void* cache, int64_t sb, int64_t sn, int64_t sh, int j) {
    int64_t row;
    if (a.block_table != nullptr) {
      int pg = a.block_table[(int64_t)b * a.max_pages + j / a.page_size];
      pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      row = pg * sb + (int64_t)(j % a.page_size) * sn;
    } else {
      row = b * sb + (int64_t)j * sn;
    }
    return (const char*)cache + (row + hk * sh) * ES;
  };
  // one 32-key block: lane l32's key, head-dim chunks ks*16 + hl*8 (keys past the split read 0,
  // so that their P = 0 meets V = 0)
  auto load_block = [&](int j0, i32x4 (&kr)[KS], i32x4 (&vr)[KS]) {
    const int j = j0 + l32;
    const bool ok = j < k_end;
    const char* ka = row_addr(a.kc, a.k_b, a.k_n, a.k_h, ok ? j : 0);
    const char* va = row_addr(a.vc, a.v_b, a.v_n, a.v_h, ok ? j : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[ks] = ok ? *(const i32x4*)(ka + (ks * 16 + hl * 8) * ES) : i32x4{};
      vr[ks] = ok ? *(const i32x4*)(va + (ks * 16 + hl * 8) * ES) : i32x4{};
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

  i32x4 kc[KS], vc[KS];
  if (jb < je) load_block(jb, kc, vc);
  for (int j0 = jb; j0 < je; j0 += 32) {
    // V(j0) into the wave's tile (row l32, chunk 2 ks + hl); the wave's own later transpose reads
    // are ordered after these writes by the LDS queue
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *(__attribute__((address_space(3))) i32x4*)(uintptr_t)(vt + T::row_off(l32, ks, hl)) = vc[ks];
    i32x4 kn[KS], vn[KS];
    const bool more = j0 + 32 < je;
    if (more) load_block(j0 + 32, kn, vn);

    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = TR::mfma(kc[ks], qop[ks], sc);
    // accumulator r: key j0 + (r/4)*8 + hl*4 + r%4 for this lane's row
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
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kc[ks] = kn[ks];
        vc[ks] = vn[ks];
      }
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
  hipLaunchKernelGGL((fa_decode_kernel<TR, D>), dim3((unsigned)units), dim3(64), 0, stream, a);
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
