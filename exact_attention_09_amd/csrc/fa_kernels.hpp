// fa_kernels.hpp — kernel arguments and launch entry points shared by the C ABI and the kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fa_schedule.hpp"

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
  // Packed variable-length batch (null for the dense [B, N, H, D] layout): sequence b is query
  // rows cu_q[b] .. cu_q[b+1]-1 of [total_q, Hq, D] and key rows cu_k[b] .. cu_k[b+1]-1 of
  // [total_k, Hkv, D]; the *_b strides are unused, Nq is the longest query sequence, and lse is
  // [Hq, total_q].
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // Block-sparse (null for dense): block_mask[hm, qb, kb] != 0 admits the pairs of query block qb
  // (kSparseBlockQ rows) and key block kb (kSparseBlockK keys); hm = 0 when mask_heads == 1, else
  // the query head.
  const uint8_t* block_mask;
  int mask_heads, nqb, nkb;
  Schedule sched;        // the launch order (make_schedule over the grid, num_q_tiles, Hq, group)
};
constexpr int kSparseBlockQ = 128;
constexpr int kSparseBlockK = 64;

// One workgroup's sequence: its sizes, the element offsets of its row 0 in q, k, v and out (head
// offsets not included), the lse index of its row 0 for query head h, and its heads' byte spans.
struct SeqView {
  int Nq, Nk;
  int64_t q0, k0, v0, o0, lse0;
  uint32_t q_bytes, k_bytes, v_bytes, o_bytes;
};

// es / oes: bytes per element of the inputs / of out. Offsets read from the device are clamped
// into [0, total], so every access stays inside the packed tensors whatever they hold.
__device__ inline SeqView seq_view(const FwdArgs& a, int b, int h, int D, int es, int oes) {
  SeqView s;
  if (a.cu_q == nullptr) {
    s.Nq = a.Nq;
    s.Nk = a.Nk;
    s.q0 = b * a.q_b;
    s.k0 = b * a.k_b;
    s.v0 = b * a.v_b;
    s.o0 = b * a.o_b;
    s.lse0 = ((int64_t)b * a.Hq + h) * a.Nq;
    s.q_bytes = a.q_bytes;
    s.k_bytes = a.k_bytes;
    s.v_bytes = a.v_bytes;
    s.o_bytes = a.o_bytes;
    return s;
  }
  auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
  const int qs = clampi(a.cu_q[b], 0, a.total_q), qe = clampi(a.cu_q[b + 1], qs, a.total_q);
  const int ks = clampi(a.cu_k[b], 0, a.total_k), ke = clampi(a.cu_k[b + 1], ks, a.total_k);
  s.Nq = qe - qs;
  s.Nk = ke - ks;
  s.q0 = qs * a.q_n;
  s.k0 = ks * a.k_n;
  s.v0 = ks * a.v_n;
  s.o0 = qs * a.o_n;
  s.lse0 = (int64_t)h * a.total_q + qs;
  auto span = [&](int n, int64_t row, int e) { return n > 0 ? (uint32_t)(((n - 1) * row + D) * e) : 0u; };
  s.q_bytes = span(s.Nq, a.q_n, es);
  s.k_bytes = span(s.Nk, a.k_n, es);
  s.v_bytes = span(s.Nk, a.v_n, es);
  s.o_bytes = span(s.Nq, a.o_n, oes);
  return s;
}

// Backward pass: one launch of the dq kernel (which also forms delta), then of the dk/dv kernel
// (and, when query heads are split, of the reduce kernel).
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
  Schedule sched_q;      // launch order of the dq kernel: its grid, num_q_tiles, Hq
  Schedule sched_k;      // of the dk/dv kernel: its grid, num_k_tiles, Hkv * n_split
};

// Queries against a dense or paged key/value cache (decode-shaped: few queries, long keys), split
// over the keys; one wave per workgroup.
struct DecArgs {
  const void* q;             // [B, Nq, Hq, D]
  const void* kc;            // dense [B, max_seqlen_k, Hkv, D], or paged [num_pages, page_size, Hkv, D]
  const void* vc;
  void* o;                   // [B, Nq, Hq, D]
  float* lse;                // [B, Hq, Nq] or null
  const int* seqlens_k;      // [B]
  const int* block_table;    // [B, max_pages] page ids, or null for a dense cache
  float* part;               // n_split > 1: fp32 outputs [n_split, B * Hq * Nq, D], then lse [n_split, B * Hq * Nq]
  int B, Nq, Hq, Hkv, group, max_seqlen_k, page_size, max_pages, num_pages;
  int causal, wl, wr;
  int row_blocks;            // ceil(group * Nq / 32): the group's query rows, 32 per wave
  int n_split, split_keys;   // splits per (batch, K/V head, row block); keys per split (a multiple of 32)
  int pages_per_split;       // paged: page ids one split can span (split_keys / page_size + 2)
  int64_t q_b, q_n, q_h, k_b, k_n, k_h, v_b, v_n, v_h, o_b, o_n, o_h;   // k_b, v_b: page stride when paged
  float scale_log2;
};
hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream);

constexpr int kBwdQRows = 128;   // query rows per dq workgroup
constexpr int kBwdKRows = 128;   // keys per dk/dv workgroup
hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream);

// Tile shapes of the launch for head dimension D and storage type.
struct TileShape {
  int block_m, block_n, waves, qb, lds_bytes;   // qb: query blocks of 32 rows per wave
  int hp;   // query heads per workgroup (they share a K/V head); block_m rows of each
};

// Whether a fp16/bf16 call takes the few-keys launch shape (4-wave workgroups, 32-key tiles):
// every row admits at most kShortRowKeys keys (a window) and the call is dense or packed, not
// block-sparse.
constexpr int kShortRowKeys = 4096;
bool short_rows(int D, int dtype, int causal, int wl, int wr, bool sparse);
TileShape tile_shape(int D, int dtype, bool few_keys, bool sparse, int group);
hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, const TileShape& ts, int64_t grid, hipStream_t stream);

}  // namespace fa
