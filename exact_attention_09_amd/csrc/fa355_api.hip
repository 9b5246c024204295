// fa355_api.hip — the C ABI of libfa355: argument validation, launch planning and dispatch.
//
// The entry point follows the pages' interface ("Flash Attention - Fast Memory-Efficient
// Attention", skill page, Workflow 2 Steps 2-3: q, k, v in [batch, seqlen, nheads, headdim],
// causal, window_size = (left, right), softmax_scale, fewer K/V heads; Workflow 3: fp8 e4m3
// inputs). Every argument is checked here, before any device call; nothing is allocated.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa355.h"
#include "fa_kernels.hpp"
#include "fa_schedule.hpp"
#include "fa_mask.hpp"

namespace fa {
hipError_t launch_fwd_f16(const FwdArgs& a, int D, int dtype, int block_n, int qb, int hp, int64_t grid,
                          hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdArgs& a, int D, int64_t grid, hipStream_t stream);

bool short_rows(int D, int dtype, int causal, int wl, int wr, bool sparse) {
  if (dtype == FA_FP8_E4M3 || sparse || wl < 0) return false;
  const int right = causal ? 0 : wr;
  return right >= 0 && (int64_t)wl + right + 1 <= kShortRowKeys;
}

TileShape tile_shape(int D, int dtype, bool few_keys, bool sparse, int group) {
  TileShape t;
  // fp16/bf16 at D = 128: 8 waves (two per SIMD, the register budget allows no more) and 64-key
  // tiles, one workgroup per compute unit. fp16/bf16 at D = 64: 4 waves of two 32-row query
  // blocks each (256 rows) against 32-key tiles: every K and V operand read from LDS serves both
  // blocks, which halves the LDS reads and the HBM -> LDS bytes per product. fp8 and block-sparse
  // calls: 4 waves of one block against 64-key tiles. Rows that admit few keys (a window) make
  // short workgroups whose pipeline start and end dominate; there, fp16/bf16 calls take 4 waves
  // of one block with 32-key tiles (half the LDS and fewer registers), so that more workgroups
  // share a compute unit and overlap (two at D = 128, three at D = 64).
  const bool f16 = dtype != FA_FP8_E4M3;
  const bool wide = f16 && D == 128 && !few_keys;
  t.waves = wide ? 8 : 4;
  t.qb = (f16 && D == 64 && !few_keys && !sparse) ? 2 : 1;
  // Few-keys calls with 4-way (or wider) GQA put 4 query heads of one K/V head in a workgroup,
  // one wave each over the same 32 rows: each K/V tile brought into LDS serves all four, and the
  // workgroup visits the 32 rows' key tiles only (a 128-row workgroup visits 3 more, which each
  // of its waves skips or masks).
  t.hp = (f16 && (few_keys || wide) && !sparse && group % 4 == 0) ? 4 : 1;
  t.block_m = 32 * t.waves * t.qb / t.hp;
  t.block_n = (f16 && (few_keys || t.qb == 2)) ? 32 : 64;
  const int es = dtype == FA_FP8_E4M3 ? 1 : 2;
  t.lds_bytes = (3 + 3) * t.block_n * D * es;   // three-slot K and V rings
  return t;
}

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, const TileShape& ts, int64_t grid, hipStream_t stream) {
  if (dtype == FA_FP8_E4M3) return launch_fwd_fp8(a, D, grid, stream);
  return launch_fwd_f16(a, D, dtype, ts.block_n, ts.qb, ts.hp, grid, stream);
}
}  // namespace fa

namespace {

constexpr int kMaxSeq = 1 << 30;
constexpr int kMaxSparseKeyBlocks = 4096;   // block-sparse: key blocks of one row (LDS tile list)
constexpr int64_t kMaxSpan = (int64_t)1 << 31;
constexpr int kSpanSlack = 256;  // rows a tile may reach past the end of a sequence

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

int elem_bytes(int dtype) { return dtype == FA_FP8_E4M3 ? 1 : 2; }

fa_status check_sizes(int B, int Nq, int Nk, int Hq, int Hkv, int D, int wl, int wr, int dtype) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_DTYPE;
  if (B < 1 || Nq < 1 || Nk < 1 || Hq < 1 || Hkv < 1) return FA_ERR_SHAPE;
  if (Nq > kMaxSeq || Nk > kMaxSeq || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (wl < -1 || wr < -1) return FA_ERR_WINDOW;
  const int64_t tiles = ((int64_t)Nq + 127) / 128;   // 128 rows: the smallest query tile
  if ((int64_t)B * Hq * tiles >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Bytes one head of a tensor spans (rows 0..n-1) and the check that a tile reaching kSpanSlack
// rows past the end still addresses it with 32-bit offsets.
bool span_ok(int64_t n, int64_t row_stride, int D, int es, uint32_t* bytes) {
  const int64_t span = ((n - 1) * row_stride + D) * es;
  const int64_t reach = ((n + kSpanSlack) * row_stride + D) * es;
  if (span >= kMaxSpan || reach >= kMaxSpan) return false;
  *bytes = (uint32_t)span;
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

namespace {

// Workgroups over which the dk/dv kernel splits the query heads of each K/V head: doubled (while
// it divides the group) until the launch has kBwdMinGrid workgroups, so that few K/V heads
// (MQA, GQA) with short keys still fill the chip.
constexpr int64_t kBwdMinGrid = 2048;
int bwd_split(int B, int Hkv, int num_k_tiles, int group) {
  const int64_t base = (int64_t)B * Hkv * num_k_tiles;
  int n = 1;
  while (base * n < kBwdMinGrid && group % (2 * n) == 0) n *= 2;
  return n;
}

// fp32 values of the backward workspace: two per query row, then (from a 16-byte boundary) dk
// and dv partial sums per split when the query heads are split.
int64_t bwd_rows_floats(int B, int Nq, int Hq) { return (2 * (int64_t)B * Hq * Nq + 3) / 4 * 4; }
int64_t bwd_workspace_floats(int B, int Nq, int Nk, int Hq, int Hkv, int D) {
  const int ns = bwd_split(B, Hkv, (Nk + fa::kBwdKRows - 1) / fa::kBwdKRows, Hq / Hkv);
  int64_t f = bwd_rows_floats(B, Nq, Hq);
  if (ns > 1) f += 2 * (int64_t)ns * B * Hkv * Nk * D;
  return f;
}

}  // namespace

namespace {

// Key splits of fa_fwd_kvcache: enough waves to cover the chip several times over (one wave per
// (batch, K/V head, row block, split)), splits of kDecMinKeys to kDecMaxKeys keys, a multiple of 32
// (the lower bound keeps a wave's fixed costs small against its streaming, the upper bound keeps a
// split's page ids within a few KB of LDS). Measured on 128 sequences of 512-8192 keys (1024
// pairs: 1024-key splits) and on 16 sequences of 4096-16384 keys (128 pairs: 512-key splits).
constexpr int64_t kDecTargetWaves = 8192;
constexpr int kDecMinKeys = 512;
constexpr int kDecMaxKeys = 4096;
void dec_split(int B, int Hkv, int row_blocks, int max_seqlen_k, int* n_split, int* split_keys) {
  const int64_t base = (int64_t)B * Hkv * row_blocks;
  const int64_t want = (kDecTargetWaves + base - 1) / base;
  int64_t keys = ((int64_t)max_seqlen_k + want - 1) / want;
  keys = keys < kDecMinKeys ? kDecMinKeys : (keys + 31) / 32 * 32;
  keys = keys > kDecMaxKeys ? kDecMaxKeys : keys;
  *split_keys = (int)keys;
  *n_split = (int)(((int64_t)max_seqlen_k + keys - 1) / keys);
}

int64_t dec_workspace_floats(int B, int Nq, int Hq, int Hkv, int D, int max_seqlen_k) {
  const int row_blocks = ((Hq / Hkv) * Nq + 31) / 32;
  int ns, sk;
  dec_split(B, Hkv, row_blocks, max_seqlen_k, &ns, &sk);
  return ns > 1 ? (int64_t)ns * B * Hq * Nq * (D + 1) : 0;
}

fa_status check_kvcache_sizes(int B, int Nq, int Hq, int Hkv, int D, int max_seqlen_k) {
  if (B < 1 || Nq < 1 || Hq < 1 || Hkv < 1 || max_seqlen_k < 1) return FA_ERR_SHAPE;
  if (Nq > kMaxSeq || max_seqlen_k > kMaxSeq || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if ((int64_t)(Hq / Hkv) * Nq > kMaxSeq) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  const int64_t row_blocks = ((int64_t)(Hq / Hkv) * Nq + 31) / 32;
  int ns, sk;
  dec_split(B, Hkv, (int)(row_blocks < kMaxSeq ? row_blocks : kMaxSeq), max_seqlen_k, &ns, &sk);
  if ((int64_t)B * Hkv * row_blocks * ns >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if ((int64_t)B * Hq * Nq * (D / 8) >= ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid sizes (B, Nq, Nk, Hq, Hkv >= 1, Hq % Hkv == 0, sizes <= 2^30)";
    case FA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case FA_ERR_WINDOW: return "window bounds must be -1 (unbounded) or >= 0";
    case FA_ERR_SCALE: return "softmax_scale and descales must be finite and > 0 (fa_bwd: softmax_scale >= 2^-120)";
    case FA_ERR_STRIDES: return "invalid strides or alignment (16-byte aligned, rows must not overlap)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_DESCALE: return "fp8 e4m3 needs descale_qkv";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_TOO_LARGE: return "one head of a tensor spans 2^31 bytes or more";
    case FA_ERR_WORKSPACE: return "workspace smaller than the sizes need (fa_bwd_workspace_bytes, fa_fwd_kvcache_workspace_bytes)";
    case FA_ERR_SCRATCH: return "the sizes need more split scratch than fa_fwd_kvcache_noalloc's fixed FA_NOALLOC_SCRATCH_BYTES";
  }
  return "unknown status";
}

fa_status fa_kv_tile_range(int Nq, int Nk, int causal, int window_left, int window_right, int block_n,
                           int row_begin, int row_end, int* tile_begin, int* tile_end, int* full, int* partial,
                           int* skipped) {
  if (!tile_begin || !tile_end) return FA_ERR_NULL;
  if (Nq < 1 || Nk < 1 || Nq > kMaxSeq || Nk > kMaxSeq || block_n < 1) return FA_ERR_SHAPE;
  if (row_begin < 0 || row_end > Nq || row_begin >= row_end) return FA_ERR_SHAPE;
  if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
  const fa::MaskSpec ms{Nq, Nk, causal ? 1 : 0, window_left, window_right};
  fa::tile_range(ms, row_begin, row_end - 1, block_n, tile_begin, tile_end);
  int nf = 0, np = 0, ns = 0;
  for (int t = *tile_begin; t < *tile_end; ++t) {
    const int c = fa::classify_tile(ms, row_begin, row_end - 1, t * block_n, block_n);
    nf += c == fa::TILE_FULL;
    np += c == fa::TILE_PARTIAL;
    ns += c == fa::TILE_SKIP;
  }
  if (full) *full = nf;
  if (partial) *partial = np;
  if (skipped) *skipped = ns;
  return FA_OK;
}

fa_status fa_block_order(int64_t n, int num_tiles, int heads, int group, int causal, int packed, int* b, int* h,
                         int* t) {
  if (!b || !h || !t) return FA_ERR_NULL;
  if (n < 1 || n >= ((int64_t)1 << 31) || num_tiles < 1 || heads < 1 || group < 1 || heads % group != 0 ||
      n % ((int64_t)heads * num_tiles) != 0)
    return FA_ERR_SHAPE;
  const fa::Schedule S = fa::make_schedule((int)n, num_tiles, heads, group, causal != 0, packed != 0);
  for (int id = 0; id < (int)n; ++id) fa::schedule_block(id, S, &b[id], &h[id], &t[id]);
  return FA_OK;
}

fa_status fa_fwd_plan(int B, int Nq, int Nk, int Hq, int Hkv, int D, int causal, int window_left, int window_right,
                      fa_dtype dtype, fa_plan_info* info) {
  if (!info) return FA_ERR_NULL;
  const fa_status st = check_sizes(B, Nq, Nk, Hq, Hkv, D, window_left, window_right, dtype);
  if (st != FA_OK) return st;
  const fa::TileShape ts =
      fa::tile_shape(D, dtype, fa::short_rows(D, dtype, causal, window_left, window_right, false), false, Hq / Hkv);
  info->block_m = ts.block_m;
  info->block_n = ts.block_n;
  info->waves = ts.waves;
  info->heads_per_wg = ts.hp;
  info->num_q_tiles = (Nq + ts.block_m - 1) / ts.block_m;
  info->grid = (int64_t)B * (Hq / ts.hp) * info->num_q_tiles;
  info->lds_bytes = ts.lds_bytes;
  const fa::MaskSpec ms{Nq, Nk, causal ? 1 : 0, window_left, window_right};
  int64_t tiles = 0;
  for (int qt = 0; qt < info->num_q_tiles; ++qt) {
    int tb, te;
    const int r0 = qt * ts.block_m, r1 = (r0 + ts.block_m < Nq ? r0 + ts.block_m : Nq) - 1;
    fa::tile_range(ms, r0, r1, ts.block_n, &tb, &te);
    tiles += te - tb;
  }
  info->kv_tiles = tiles * B * (Hq / ts.hp);
  return FA_OK;
}

}  // extern "C"

namespace {

// fa_fwd, and fa_fwd_blocksparse when block_mask is set.
fa_status fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Nq, int Nk, int Hq,
                   int Hkv, int D, const fa_strides* s, float softmax_scale, int causal, int window_left,
                   int window_right, fa_dtype dtype, hipStream_t stream, const float* descale_qkv,
                   const uint8_t* block_mask, int mask_heads) {
  if (!q || !k || !v || !out || !s) return FA_ERR_NULL;
  fa_status st = check_sizes(B, Nq, Nk, Hq, Hkv, D, window_left, window_right, dtype);
  if (st != FA_OK) return st;
  if (!finite_pos(softmax_scale)) return FA_ERR_SCALE;
  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (dtype == FA_FP8_E4M3) {
    if (!descale_qkv) return FA_ERR_DESCALE;
    dq = descale_qkv[0];
    dk = descale_qkv[1];
    dv = descale_qkv[2];
    if (!finite_pos(dq) || !finite_pos(dk) || !finite_pos(dv)) return FA_ERR_SCALE;
  }
  const int es = elem_bytes(dtype);
  const int oes = 2;
  // strides: non-negative; output rows and heads must not overlap; 16-byte alignment
  const int64_t in_str[9] = {s->q_b, s->q_n, s->q_h, s->k_b, s->k_n, s->k_h, s->v_b, s->v_n, s->v_h};
  for (int i = 0; i < 9; ++i)
    if (in_str[i] < 0 || (in_str[i] * es) % 16 != 0) return FA_ERR_STRIDES;
  const int64_t out_str[3] = {s->o_b, s->o_n, s->o_h};
  for (int i = 0; i < 3; ++i)
    if (out_str[i] < 0 || (out_str[i] * oes) % 16 != 0) return FA_ERR_STRIDES;
  if ((Nq > 1 && s->o_n < D) || (Hq > 1 && s->o_h < D) || (B > 1 && s->o_b < D)) return FA_ERR_STRIDES;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)lse & 3u)) return FA_ERR_STRIDES;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.B = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.q_b = s->q_b; a.q_n = s->q_n; a.q_h = s->q_h;
  a.k_b = s->k_b; a.k_n = s->k_n; a.k_h = s->k_h;
  a.v_b = s->v_b; a.v_n = s->v_n; a.v_h = s->v_h;
  a.o_b = s->o_b; a.o_n = s->o_n; a.o_h = s->o_h;
  if (!span_ok(Nq, s->q_n, D, es, &a.q_bytes) || !span_ok(Nk, s->k_n, D, es, &a.k_bytes) ||
      !span_ok(Nk, s->v_n, D, es, &a.v_bytes) || !span_ok(Nq, s->o_n, D, oes, &a.o_bytes))
    return FA_ERR_TOO_LARGE;
  const double log2e = 1.4426950408889634074;
  a.scale_log2 = (float)((double)softmax_scale * dq * dk * log2e);
  a.out_scale = dtype == FA_FP8_E4M3 ? dv : 1.f;
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.block_mask = block_mask;
  a.mask_heads = mask_heads;
  a.nqb = (Nq + fa::kSparseBlockQ - 1) / fa::kSparseBlockQ;
  a.nkb = (Nk + fa::kSparseBlockK - 1) / fa::kSparseBlockK;
  const bool sparse = block_mask != nullptr;
  const fa::TileShape ts =
      fa::tile_shape(D, dtype, fa::short_rows(D, dtype, causal, window_left, window_right, sparse), sparse, a.group);
  a.num_q_tiles = (Nq + ts.block_m - 1) / ts.block_m;
  const int64_t grid = (int64_t)B * (Hq / ts.hp) * a.num_q_tiles;
  a.sched = fa::make_schedule((int)grid, a.num_q_tiles, Hq / ts.hp, a.group / ts.hp, causal != 0, false);
  const hipError_t e = fa::launch_fwd(a, D, dtype, ts, grid, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Nq, int Nk, int Hq,
                 int Hkv, int D, const fa_strides* s, float softmax_scale, int causal, int window_left,
                 int window_right, fa_dtype dtype, hipStream_t stream, const float* descale_qkv) {
  return fwd_impl(q, k, v, out, lse, B, Nq, Nk, Hq, Hkv, D, s, softmax_scale, causal, window_left, window_right,
                  dtype, stream, descale_qkv, nullptr, 0);
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Nq,
                             int Nk, int Hq, int Hkv, int D, const fa_strides* s, float softmax_scale, int causal,
                             int window_left, int window_right, fa_dtype dtype, hipStream_t stream,
                             const uint8_t* block_mask, int mask_heads) {
  if (!block_mask) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask_heads != 1 && mask_heads != Hq) return FA_ERR_SHAPE;
  // the tile list of a workgroup lives in LDS next to the K/V rings
  if ((int64_t)Nk > (int64_t)kMaxSparseKeyBlocks * fa::kSparseBlockK) return FA_ERR_SHAPE;
  return fwd_impl(q, k, v, out, lse, B, Nq, Nk, Hq, Hkv, D, s, softmax_scale, causal, window_left, window_right,
                  dtype, stream, nullptr, block_mask, mask_heads);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int B, int total_q, int total_k, int max_seqlen_q, int Hq,
                        int Hkv, int D, const fa_varlen_strides* s, float softmax_scale, int causal,
                        int window_left, int window_right, fa_dtype dtype, hipStream_t stream,
                        const float* descale_qkv) {
  if (!q || !k || !v || !out || !s || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  // the sizes as one dense launch of B sequences of max_seqlen_q queries
  fa_status st = check_sizes(B, max_seqlen_q, total_k, Hq, Hkv, D, window_left, window_right, dtype);
  if (st != FA_OK) return st;
  if (total_q < 1 || total_q > kMaxSeq || max_seqlen_q > total_q) return FA_ERR_SHAPE;
  if (!finite_pos(softmax_scale)) return FA_ERR_SCALE;
  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (dtype == FA_FP8_E4M3) {
    if (!descale_qkv) return FA_ERR_DESCALE;
    dq = descale_qkv[0];
    dk = descale_qkv[1];
    dv = descale_qkv[2];
    if (!finite_pos(dq) || !finite_pos(dk) || !finite_pos(dv)) return FA_ERR_SCALE;
  }
  const int es = elem_bytes(dtype);
  const int oes = 2;
  const int64_t in_str[6] = {s->q_n, s->q_h, s->k_n, s->k_h, s->v_n, s->v_h};
  for (int i = 0; i < 6; ++i)
    if (in_str[i] < 0 || (in_str[i] * es) % 16 != 0) return FA_ERR_STRIDES;
  if (s->o_n < 0 || s->o_h < 0 || (s->o_n * oes) % 16 != 0 || (s->o_h * oes) % 16 != 0) return FA_ERR_STRIDES;
  if ((total_q > 1 && s->o_n < D) || (Hq > 1 && s->o_h < D)) return FA_ERR_STRIDES;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)lse & 3u)) return FA_ERR_STRIDES;
  if (((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u)) return FA_ERR_STRIDES;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.B = B;
  a.Nq = max_seqlen_q;
  a.Nk = total_k;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.q_b = a.k_b = a.v_b = a.o_b = 0;
  a.q_n = s->q_n; a.q_h = s->q_h;
  a.k_n = s->k_n; a.k_h = s->k_h;
  a.v_n = s->v_n; a.v_h = s->v_h;
  a.o_n = s->o_n; a.o_h = s->o_h;
  // every sequence is a row range of the packed tensors: bound the whole packed span
  if (!span_ok(total_q, s->q_n, D, es, &a.q_bytes) || !span_ok(total_k, s->k_n, D, es, &a.k_bytes) ||
      !span_ok(total_k, s->v_n, D, es, &a.v_bytes) || !span_ok(total_q, s->o_n, D, oes, &a.o_bytes))
    return FA_ERR_TOO_LARGE;
  const double log2e = 1.4426950408889634074;
  a.scale_log2 = (float)((double)softmax_scale * dq * dk * log2e);
  a.out_scale = dtype == FA_FP8_E4M3 ? dv : 1.f;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.block_mask = nullptr;
  a.mask_heads = a.nqb = a.nkb = 0;
  a.total_q = total_q;
  a.total_k = total_k;
  const fa::TileShape ts =
      fa::tile_shape(D, dtype, fa::short_rows(D, dtype, causal, window_left, window_right, false), false, a.group);
  a.num_q_tiles = (max_seqlen_q + ts.block_m - 1) / ts.block_m;
  const int64_t grid = (int64_t)B * (Hq / ts.hp) * a.num_q_tiles;
  a.sched = fa::make_schedule((int)grid, a.num_q_tiles, Hq / ts.hp, a.group / ts.hp, causal != 0, true);
  const hipError_t e = fa::launch_fwd(a, D, dtype, ts, grid, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_fwd_kvcache_workspace_bytes(int B, int Nq, int Hq, int Hkv, int D, int max_seqlen_k) {
  if (check_kvcache_sizes(B, Nq, Hq, Hkv, D, max_seqlen_k) != FA_OK) return 0;
  return (size_t)dec_workspace_floats(B, Nq, Hq, Hkv, D, max_seqlen_k) * 4u;
}

}  // extern "C"

// The fixed scratch of fa_fwd_kvcache_noalloc: one copy per GPU in the library's device code,
// held until the process ends. Host code never uses the array's name as an address (on the host
// it only stands for the symbol): the device address comes from hipGetSymbolAddress, resolved
// once per device with that device current, and kept per device (scratch_ptr below).
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// fa_fwd_kvcache, and fa_fwd_kvcache_noalloc when scratch_call is set: then `workspace` is not
// known yet; it is resolved (scratch_ptr) after every argument check, and a need above
// FA_NOALLOC_SCRATCH_BYTES is FA_ERR_SCRATCH.
void* scratch_ptr();
fa_status kvcache_impl(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                       const int32_t* seqlens_k, const int32_t* block_table, int B, int Nq, int Hq, int Hkv, int D,
                       int max_seqlen_k, int page_size, int max_pages_per_seq, int num_pages, const fa_strides* s,
                       float softmax_scale, int causal, int window_left, int window_right, fa_dtype dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream, bool scratch_call) {
  if (!q || !k_cache || !v_cache || !out || !seqlens_k || !s) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  fa_status st = check_kvcache_sizes(B, Nq, Hq, Hkv, D, max_seqlen_k);
  if (st != FA_OK) return st;
  if (block_table != nullptr && (page_size < 1 || max_pages_per_seq < 1 || num_pages < 1)) return FA_ERR_SHAPE;
  if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
  if (!finite_pos(softmax_scale)) return FA_ERR_SCALE;
  const int64_t need = dec_workspace_floats(B, Nq, Hq, Hkv, D, max_seqlen_k) * 4;
  if (scratch_call) {
    if ((uint64_t)need > (uint64_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    workspace_bytes = FA_NOALLOC_SCRATCH_BYTES;
    workspace = nullptr;   // resolved below, once the other arguments are known to be valid
  } else if ((uint64_t)workspace_bytes < (uint64_t)need || (need > 0 && workspace == nullptr)) {
    return FA_ERR_WORKSPACE;
  }
  const int64_t str[12] = {s->q_b, s->q_n, s->q_h, s->k_b, s->k_n, s->k_h, s->v_b, s->v_n, s->v_h, s->o_b, s->o_n, s->o_h};
  for (int i = 0; i < 12; ++i)
    if (str[i] < 0 || (str[i] * 2) % 16 != 0) return FA_ERR_STRIDES;
  if ((Nq > 1 && s->o_n < D) || (Hq > 1 && s->o_h < D) || (B > 1 && s->o_b < D)) return FA_ERR_STRIDES;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(workspace) ||
      ((uintptr_t)lse & 3u) || ((uintptr_t)seqlens_k & 3u) || ((uintptr_t)block_table & 3u))
    return FA_ERR_STRIDES;
  if (scratch_call && need > 0) {
    workspace = scratch_ptr();
    if (workspace == nullptr) return FA_ERR_LAUNCH;
  }

  fa::DecArgs a;
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.o = out; a.lse = lse;
  a.seqlens_k = seqlens_k;
  a.block_table = block_table;
  a.part = (float*)workspace;
  a.B = B; a.Nq = Nq; a.Hq = Hq; a.Hkv = Hkv; a.group = Hq / Hkv;
  a.max_seqlen_k = max_seqlen_k;
  a.page_size = block_table ? page_size : 0;
  a.max_pages = block_table ? max_pages_per_seq : 0;
  a.num_pages = block_table ? num_pages : 0;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.row_blocks = (a.group * Nq + 31) / 32;
  dec_split(B, Hkv, a.row_blocks, max_seqlen_k, &a.n_split, &a.split_keys);
  a.pages_per_split = block_table ? a.split_keys / page_size + 2 : 0;
  a.q_b = s->q_b; a.q_n = s->q_n; a.q_h = s->q_h;
  a.k_b = s->k_b; a.k_n = s->k_n; a.k_h = s->k_h;
  a.v_b = s->v_b; a.v_n = s->v_n; a.v_h = s->v_h;
  a.o_b = s->o_b; a.o_n = s->o_n; a.o_h = s->o_h;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  const hipError_t e = fa::launch_decode(a, D, dtype, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (resolved on the first call on that device), or null if it
// cannot be resolved.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

fa_status fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                         const int32_t* seqlens_k, const int32_t* block_table, int B, int Nq, int Hq, int Hkv, int D,
                         int max_seqlen_k, int page_size, int max_pages_per_seq, int num_pages, const fa_strides* s,
                         float softmax_scale, int causal, int window_left, int window_right, fa_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kvcache_impl(q, k_cache, v_cache, out, lse, seqlens_k, block_table, B, Nq, Hq, Hkv, D, max_seqlen_k,
                      page_size, max_pages_per_seq, num_pages, s, softmax_scale, causal, window_left, window_right,
                      dtype, workspace, workspace_bytes, stream, false);
}

fa_status fa_fwd_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                 const int32_t* seqlens_k, const int32_t* block_table, int B, int Nq, int Hq,
                                 int Hkv, int D, int max_seqlen_k, int page_size, int max_pages_per_seq,
                                 int num_pages, const fa_strides* s, float softmax_scale, int causal,
                                 int window_left, int window_right, fa_dtype dtype, hipStream_t stream) {
  return kvcache_impl(q, k_cache, v_cache, out, lse, seqlens_k, block_table, B, Nq, Hq, Hkv, D, max_seqlen_k,
                      page_size, max_pages_per_seq, num_pages, s, softmax_scale, causal, window_left, window_right,
                      dtype, nullptr, 0, stream, true);
}

size_t fa_bwd_workspace_bytes(int B, int Nq, int Nk, int Hq, int Hkv, int D) {
  if (check_sizes(B, Nq, Nk, Hq, Hkv, D, -1, -1, FA_F16) != FA_OK) return 0;
  return (size_t)bwd_workspace_floats(B, Nq, Nk, Hq, Hkv, D) * 4u;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Nq, int Nk, int Hq,
                 int Hkv, int D, const fa_bwd_strides* s, float softmax_scale, int causal, int window_left,
                 int window_right, fa_dtype dtype, hipStream_t stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace || !s) return FA_ERR_NULL;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  fa_status st = check_sizes(B, Nq, Nk, Hq, Hkv, D, window_left, window_right, dtype);
  if (st != FA_OK) return st;
  if ((uint64_t)workspace_bytes < (uint64_t)bwd_workspace_floats(B, Nq, Nk, Hq, Hkv, D) * 4u) return FA_ERR_WORKSPACE;
  // the workspace holds lse / softmax_scale: bounded scales keep it finite
  if (!finite_pos(softmax_scale) || softmax_scale < 0x1p-120f) return FA_ERR_SCALE;
  const int64_t str[24] = {s->q_b,  s->q_n,  s->q_h,  s->k_b,  s->k_n,  s->k_h,  s->v_b,  s->v_n,
                           s->v_h,  s->o_b,  s->o_n,  s->o_h,  s->do_b, s->do_n, s->do_h, s->dq_b,
                           s->dq_n, s->dq_h, s->dk_b, s->dk_n, s->dk_h, s->dv_b, s->dv_n, s->dv_h};
  for (int i = 0; i < 24; ++i)
    if (str[i] < 0 || (str[i] * 2) % 16 != 0) return FA_ERR_STRIDES;
  // written tensors: rows and heads must not overlap
  if ((Nq > 1 && s->dq_n < D) || (Hq > 1 && s->dq_h < D) || (B > 1 && s->dq_b < D)) return FA_ERR_STRIDES;
  if ((Nk > 1 && (s->dk_n < D || s->dv_n < D)) || (Hkv > 1 && (s->dk_h < D || s->dv_h < D)) ||
      (B > 1 && (s->dk_b < D || s->dv_b < D)))
    return FA_ERR_STRIDES;
  const void* ptrs[9] = {q, k, v, out, dout, dq, dk, dv, workspace};
  for (int i = 0; i < 9; ++i)
    if (!aligned16(ptrs[i])) return FA_ERR_STRIDES;
  if ((uintptr_t)lse & 3u) return FA_ERR_STRIDES;
  if ((int64_t)B * Hq * Nq >= ((int64_t)1 << 31) / 16) return FA_ERR_SHAPE;

  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = (float*)workspace;
  a.B = B; a.Nq = Nq; a.Nk = Nk; a.Hq = Hq; a.Hkv = Hkv; a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.num_q_tiles = (Nq + fa::kBwdQRows - 1) / fa::kBwdQRows;
  a.num_k_tiles = (Nk + fa::kBwdKRows - 1) / fa::kBwdKRows;
  a.n_split = bwd_split(B, Hkv, a.num_k_tiles, Hq / Hkv);
  a.part = a.delta + bwd_rows_floats(B, Nq, Hq);
  a.q_b = s->q_b; a.q_n = s->q_n; a.q_h = s->q_h;
  a.k_b = s->k_b; a.k_n = s->k_n; a.k_h = s->k_h;
  a.v_b = s->v_b; a.v_n = s->v_n; a.v_h = s->v_h;
  a.o_b = s->o_b; a.o_n = s->o_n; a.o_h = s->o_h;
  a.do_b = s->do_b; a.do_n = s->do_n; a.do_h = s->do_h;
  a.dq_b = s->dq_b; a.dq_n = s->dq_n; a.dq_h = s->dq_h;
  a.dk_b = s->dk_b; a.dk_n = s->dk_n; a.dk_h = s->dk_h;
  a.dv_b = s->dv_b; a.dv_n = s->dv_n; a.dv_h = s->dv_h;
  if (!span_ok(Nq, s->q_n, D, 2, &a.q_bytes) || !span_ok(Nk, s->k_n, D, 2, &a.k_bytes) ||
      !span_ok(Nk, s->v_n, D, 2, &a.v_bytes) || !span_ok(Nq, s->o_n, D, 2, &a.o_bytes) ||
      !span_ok(Nq, s->do_n, D, 2, &a.do_bytes) || !span_ok(Nq, s->dq_n, D, 2, &a.dq_bytes) ||
      !span_ok(Nk, s->dk_n, D, 2, &a.dk_bytes) || !span_ok(Nk, s->dv_n, D, 2, &a.dv_bytes))
    return FA_ERR_TOO_LARGE;
  if ((int64_t)B * Hkv * a.num_k_tiles * a.n_split >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  a.scale = softmax_scale;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  a.sched_q = fa::make_schedule((int)((int64_t)B * Hq * a.num_q_tiles), a.num_q_tiles, Hq, 1, causal != 0, false);
  a.sched_k = fa::make_schedule((int)((int64_t)B * Hkv * a.n_split * a.num_k_tiles), a.num_k_tiles, Hkv * a.n_split, 1,
                                causal != 0, false);
  const hipError_t e = fa::launch_bwd(a, D, dtype, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
