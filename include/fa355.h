/*
 * fa355.h — C ABI of libfa355: the FlashAttention forward pass (and its backward pass, fa_bwd)
 * on AMD MI355X (gfx950).
 *
 * What is computed ("Flash Attention - Fast Memory-Efficient Attention", skill page, Workflow 1
 * Step 2 and Workflow 2 Steps 2-3; "What FlashAttention is and how it speeds up attention",
 * sections 1-3: the fused, blocked computation is exact):
 *
 *   out[b, i, h, :] = sum_j softmax_j(s_ij) * v[b, j, g, :],
 *   s_ij = softmax_scale * <q[b, i, h, :], k[b, j, g, :]>,   g = h / (Hq / Hkv)
 *   lse[b, h, i]    = ln sum_j exp(s_ij)        (over admitted keys j only)
 *
 * in one fused kernel with an online softmax: the Nq x Nk score matrix is never written to
 * device memory. Key j is admitted for query row i when, with off = Nk - Nq,
 *   0 <= j < Nk,
 *   causal == 0 or j <= i + off                (bottom-right alignment; the usual lower
 *                                               triangle when Nq == Nk),
 *   window_left  < 0 or j >= i + off - window_left,
 *   window_right < 0 or j <= i + off + window_right.
 * A row with no admitted key gets out = 0 and lse = -inf.
 *
 * Tensors use the pages' [batch, seqlen, nheads, headdim] layout (skill page, Quick start and
 * Workflow 2 Step 2) with arbitrary element strides for batch, seqlen and heads; headdim is
 * contiguous. K and V may have fewer heads than Q (MQA / GQA, skill page, Workflow 2 Step 3):
 * query head h reads K/V head h / (Hq / Hkv).
 *
 * Storage types (skill page, Workflow 3 for fp8):
 *   FA_F16       q, k, v, out: IEEE binary16.
 *   FA_BF16      q, k, v, out: bfloat16.
 *   FA_FP8_E4M3  q, k, v: OCP fp8 E4M3 codes (max 448, no infinities) with per-tensor
 *                dequantisation scales; out: bfloat16. The score is
 *                softmax_scale * (dq * q8) . (dk * k8) and the output is sum_j p_ij * (dv * v8).
 * Arithmetic: fp32 accumulation of both products and of the softmax statistics.
 */
#ifndef FA355_H
#define FA355_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
  FA_F16 = 0,
  FA_BF16 = 1,
  FA_FP8_E4M3 = 2
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* q, k, v, out or strides is NULL (lse may be NULL)                      */
  FA_ERR_SHAPE = 2,     /* B, Nq, Nk, Hq or Hkv < 1, Hq % Hkv != 0, or a size above 2^30          */
  FA_ERR_HEAD_DIM = 3,  /* D is not 64 or 128                                                      */
  FA_ERR_WINDOW = 4,    /* window_left or window_right < -1                                       */
  FA_ERR_SCALE = 5,     /* softmax_scale not finite and > 0, or a descale not finite and > 0      */
  FA_ERR_STRIDES = 6,   /* a stride < 0, rows overlap (seqlen stride < D or head stride < D),     */
                        /* or a pointer / stride not 16-byte aligned                              */
  FA_ERR_DTYPE = 7,     /* unknown dtype                                                           */
  FA_ERR_DESCALE = 8,   /* FA_FP8_E4M3 without descale_qkv                                         */
  FA_ERR_LAUNCH = 9,    /* the kernel launch failed (HIP error; e.g. no device)                    */
  FA_ERR_TOO_LARGE = 10, /* one head's span of q, k, v or out reaches 2^31 bytes                   */
                         /* (fa_bwd: also dout, dq, dk, dv); the span counts 256 rows past the    */
                         /* head's last row, which a ragged tile's 32-bit offsets may address:    */
                         /* ((rows + 256) * row_stride + D) * element bytes < 2^31                */
  FA_ERR_WORKSPACE = 11, /* fa_bwd / fa_fwd_kvcache: workspace_bytes below what the sizes need     */
  FA_ERR_SCRATCH = 12    /* fa_fwd_kvcache_noalloc: the sizes need more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Element strides (not bytes) of the batch, seqlen and head axes; the headdim stride is 1. */
typedef struct fa_strides {
  int64_t q_b, q_n, q_h;
  int64_t k_b, k_n, k_h;
  int64_t v_b, v_n, v_h;
  int64_t o_b, o_n, o_h;
} fa_strides;

/*
 * fa_fwd — enqueue one attention forward pass on `stream`.
 *
 * q    device, [B, Nq, Hq, D] in `dtype` storage.
 * k, v device, [B, Nk, Hkv, D] in `dtype` storage.
 * out  device, [B, Nq, Hq, D]: fp16 for FA_F16, bf16 for FA_BF16 and FA_FP8_E4M3. Must not
 *      alias q, k or v.
 * lse  device fp32 [B, Hq, Nq], contiguous, natural log, scale (and fp8 descales) included;
 *      may be NULL, then it is not written.
 * softmax_scale  finite, > 0 (callers wanting the default pass 1/sqrt(D)).
 * causal         0 or 1.  window_left / window_right: -1 = unbounded, else >= 0.
 * descale_qkv    host float[3] = {dq, dk, dv}; required for FA_FP8_E4M3, ignored otherwise.
 * stream         HIP stream (0 = the null stream).
 *
 * Ownership: the caller allocates and owns every buffer. The library allocates no device
 * memory, keeps no per-call state, and is reentrant. The call is asynchronous: it returns once
 * the kernel is enqueued and never synchronises. Arguments are validated before any device call;
 * an invalid call returns its error code and touches nothing. Faults inside the kernel surface as
 * HIP errors at the caller's next synchronisation.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Nq, int Nk, int Hq, int Hkv, int D, const fa_strides* strides,
                 float softmax_scale, int causal, int window_left, int window_right,
                 fa_dtype dtype, hipStream_t stream, const float* descale_qkv);

/*
 * fa_fwd_blocksparse — fa_fwd restricted to the (query block, key block) pairs a block mask sets,
 * skipping the key tiles no row of a workgroup needs. The pages report a block-sparse variant of
 * FlashAttention that scales to 64k tokens and runs 2-4 times faster than the dense one ("What
 * FlashAttention is and how it speeds up attention", FAQ on the quadratic complexity) without an
 * interface or a pattern; this is the library's reading. Query i and key j are admitted when
 * block_mask[hm * nqb * nkb + (i / 128) * nkb + j / 64] != 0 and fa_fwd's causal / window rules
 * admit them; nqb = ceil(Nq / 128), nkb = ceil(Nk / 64); hm = 0 when mask_heads == 1, else the
 * query head. A row with no admitted key gets out = 0 and lse = -inf.
 *
 * block_mask         device uint8 [mask_heads, nqb, nkb], read by the kernel (no host copy).
 * mask_heads         1 (one mask for every head) or Hq.
 * dtype              FA_F16 or FA_BF16 (else FA_ERR_DTYPE). Nk <= 4096 * 64 (else FA_ERR_SHAPE).
 * Other arguments, validation, errors and asynchrony as for fa_fwd.
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse,
                             int B, int Nq, int Nk, int Hq, int Hkv, int D, const fa_strides* strides,
                             float softmax_scale, int causal, int window_left, int window_right,
                             fa_dtype dtype, hipStream_t stream, const uint8_t* block_mask,
                             int mask_heads);

/* Element strides of packed variable-length tensors: token and head axes (headdim stride 1). */
typedef struct fa_varlen_strides {
  int64_t q_n, q_h;
  int64_t k_n, k_h;
  int64_t v_n, v_h;
  int64_t o_n, o_h;
} fa_varlen_strides;

/*
 * fa_fwd_varlen — fa_fwd over a packed batch of B sequences of different lengths, with no
 * padding. The pages list variable sequence lengths among the ROCm backends' features ("What
 * FlashAttention is and how it speeds up attention", section "Versions, hardware and sources")
 * and describe kernels that adapt to dynamic sequence lengths without padding ("FlashAttention
 * V3 principles and practice", section 1); the interface is this library's reading.
 *
 * q                  device [total_q, Hq, D]; k, v: device [total_k, Hkv, D]; out: device
 *                    [total_q, Hq, D] (dtype rules of fa_fwd); strides in elements, headdim 1.
 * cu_seqlens_q/_k    device int32 [B + 1]: non-decreasing, from 0 to total_q / total_k. Sequence
 *                    b is query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 *                    cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1, and is computed exactly as fa_fwd
 *                    computes one sequence of those lengths (causal alignment and window use its
 *                    own lengths); a sequence with queries but no keys gives out = 0 and
 *                    lse = -inf on its rows. The offsets are read on the device (this call does
 *                    not synchronise); offsets outside [0, total] are clamped, so the kernel never
 *                    reads or writes outside the packed tensors whatever they hold.
 * max_seqlen_q       host int, 1 <= max_seqlen_q <= total_q: no sequence has more queries (rows of a
 *                    longer one past max_seqlen_q are not written).
 * lse                device fp32 [Hq, total_q] contiguous, or NULL.
 * Other arguments, validation, ownership, errors and asynchrony as for fa_fwd (total_q, total_k
 * and max_seqlen_q take the places of Nq and Nk in the size checks).
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                        int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int D,
                        const fa_varlen_strides* strides, float softmax_scale, int causal,
                        int window_left, int window_right, fa_dtype dtype, hipStream_t stream,
                        const float* descale_qkv);

/*
 * fa_fwd_kvcache — attention of Nq queries per sequence against each sequence's keys in a dense
 * or paged key/value cache: the decode-shaped workload (few queries, long keys). The pages name a
 * paged KV cache ("Flash Attention - Fast Memory-Efficient Attention", skill page, section
 * "Advanced features"; "FlashAttention V3 principles and practice", section 4, with 16-token
 * cache blocks) but no interface; this is the library's reading. Sequence b is computed exactly as
 * fa_fwd computes q[b] against Nk = seqlens_k[b] keys (bottom-right causal alignment, so with
 * Nq = 1 the query sees every key; windows as in fa_fwd); a sequence with no keys gives out = 0 and
 * lse = -inf. The keys are split over workgroups and the splits merged through the workspace.
 *
 * q, out             device [B, Nq, Hq, D] (strides q_*, o_*); fp16 or bf16, out in the same type.
 * k_cache, v_cache   device. Dense (block_table NULL): [B, max_seqlen_k, Hkv, D] with strides
 *                    (k_b, k_n, k_h). Paged: [num_pages, page_size, Hkv, D] with k_b / v_b the page
 *                    stride; key j of sequence b is slot j % page_size of page
 *                    block_table[b * max_pages_per_seq + j / page_size].
 * seqlens_k          device int32 [B]: keys of each sequence, clamped on the device to
 *                    [0, max_seqlen_k] (and to max_pages_per_seq * page_size when paged).
 * block_table        device int32 [B, max_pages_per_seq] page ids (clamped to [0, num_pages - 1]
 *                    on the device), or NULL for a dense cache (then page_size, max_pages_per_seq
 *                    and num_pages are ignored). The clamps keep every access inside the cache
 *                    whatever the device arrays hold.
 * lse                device fp32 [B, Hq, Nq] contiguous, or NULL.
 * workspace          device scratch of at least fa_fwd_kvcache_workspace_bytes(...) bytes, 16-byte
 *                    aligned, owned by the caller (may be NULL when that is 0).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (sizes < 1, Hq % Hkv, a paged cache with page_size,
 * max_pages_per_seq or num_pages < 1, or a launch too large), FA_ERR_HEAD_DIM, FA_ERR_WINDOW,
 * FA_ERR_SCALE, FA_ERR_STRIDES (negative or not 16-byte multiples, overlapping out rows, a
 * misaligned pointer), FA_ERR_DTYPE (only FA_F16 and FA_BF16), FA_ERR_WORKSPACE, FA_ERR_LAUNCH.
 * Asynchronous on `stream`; deterministic (the splits are merged in a fixed order).
 */
fa_status fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                         const int32_t* seqlens_k, const int32_t* block_table, int B, int Nq, int Hq, int Hkv,
                         int D, int max_seqlen_k, int page_size, int max_pages_per_seq, int num_pages,
                         const fa_strides* strides, float softmax_scale, int causal, int window_left,
                         int window_right, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of workspace fa_fwd_kvcache needs for these sizes (0 when the keys are not split, and for
 * invalid sizes). Pure host function. */
size_t fa_fwd_kvcache_workspace_bytes(int B, int Nq, int Hq, int Hkv, int D, int max_seqlen_k);

/* Bytes of the per-device scratch array behind fa_fwd_kvcache_noalloc (64 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fa_fwd_kvcache_noalloc — fa_fwd_kvcache for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same operation,
 * kernels, arguments (minus workspace and workspace_bytes), results (bitwise) and errors as
 * fa_fwd_kvcache. The split partials go to a fixed scratch array of FA_NOALLOC_SCRATCH_BYTES bytes
 * in the library's device code, one per GPU, which each GPU keeps until the process ends; the
 * call allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *  - Runs on the current device; its first call on a device resolves the array's address there.
 *  - FA_ERR_SCRATCH, before any device call, when fa_fwd_kvcache_workspace_bytes of the sizes
 *    exceeds FA_NOALLOC_SCRATCH_BYTES; FA_ERR_LAUNCH if the array's address cannot be resolved.
 *  - Calls on one GPU share its array: calls that overlap in time on one GPU (other streams or
 *    threads without ordering between them) race and give undefined results. Calls ordered on a
 *    stream are safe; the array keeps the last call's partials, and nothing needs clearing (each
 *    call writes every partial it reads).
 */
fa_status fa_fwd_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                 const int32_t* seqlens_k, const int32_t* block_table, int B, int Nq, int Hq,
                                 int Hkv, int D, int max_seqlen_k, int page_size, int max_pages_per_seq,
                                 int num_pages, const fa_strides* strides, float softmax_scale, int causal,
                                 int window_left, int window_right, fa_dtype dtype, hipStream_t stream);

/* Element strides of the backward pass's tensors (headdim stride 1). */
typedef struct fa_bwd_strides {
  int64_t q_b, q_n, q_h;
  int64_t k_b, k_n, k_h;
  int64_t v_b, v_n, v_h;
  int64_t o_b, o_n, o_h;        /* out of the forward pass                         */
  int64_t do_b, do_n, do_h;     /* dout: gradient of the loss w.r.t. out            */
  int64_t dq_b, dq_n, dq_h;
  int64_t dk_b, dk_n, dk_h;
  int64_t dv_b, dv_n, dv_h;
} fa_bwd_strides;

/*
 * fa_bwd — enqueue the backward pass of fa_fwd on `stream`: the gradients of a loss with respect
 * to q, k and v, given dout, the gradient of the loss with respect to out. The pages name the
 * backward pass and its recomputation of attention from the saved statistics ("Flash Attention -
 * Fast Memory-Efficient Attention", skill page, Quick start; "What FlashAttention is and how it
 * speeds up attention", section "Versions, hardware and sources"); with p_ij the softmax weights
 * of the forward pass (recomputed from q, k and lse),
 *   dv_j = sum_i p_ij dout_i,   ds_ij = p_ij (dout_i . v_j - dout_i . out_i),
 *   dq_i = softmax_scale * sum_j ds_ij k_j,   dk_j = softmax_scale * sum_i ds_ij q_i,
 * summed over the query heads that share a K/V head (MQA/GQA).
 *
 * q, k, v, out, lse  device: the forward pass's inputs and outputs for the same sizes, options
 *                    and dtype (lse is required here: fp32 [B, Hq, Nq], contiguous).
 * dout               device, [B, Nq, Hq, D], dtype storage.
 * dq                 device, [B, Nq, Hq, D];  dk, dv: device, [B, Nk, Hkv, D]; dtype storage.
 *                    Written in full (every row, including rows with no admitted key: zero).
 *                    Must not alias each other or the inputs.
 * workspace          device scratch of workspace_bytes >= fa_bwd_workspace_bytes(B, Nq, Nk, Hq,
 *                    Hkv, D) bytes (else FA_ERR_WORKSPACE), 16-byte aligned, owned by the caller;
 *                    its contents on entry do not matter. It holds two fp32 values per query row
 *                    (-rowsum(dout * out) and -lse / softmax_scale) and, when the query heads of
 *                    a K/V head are split over several workgroups (few K/V heads and short keys),
 *                    their fp32 partial sums of dk and dv, added up in a fixed order.
 * softmax_scale      finite and at least 2^-120 (else FA_ERR_SCALE), so that lse / softmax_scale
 *                    stays finite.
 * dtype              FA_F16 or FA_BF16 (FA_FP8_E4M3 returns FA_ERR_DTYPE).
 * Other arguments, validation, ownership and asynchrony as for fa_fwd. Deterministic: no
 * atomics; the same inputs give bitwise the same gradients.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int B, int Nq, int Nk, int Hq, int Hkv, int D, const fa_bwd_strides* strides,
                 float softmax_scale, int causal, int window_left, int window_right,
                 fa_dtype dtype, hipStream_t stream);

/*
 * fa_bwd_workspace_bytes — bytes of device workspace fa_bwd needs for these sizes (a multiple of
 * 4); 0 when the sizes are invalid for fa_bwd (then fa_bwd reports the reason). Pure host
 * function: no device call.
 */
size_t fa_bwd_workspace_bytes(int B, int Nq, int Nk, int Hq, int Hkv, int D);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* Launch plan of one fa_fwd call (host only, no device call). */
typedef struct fa_plan_info {
  int block_m;        /* query rows per workgroup, of each of its heads             */
  int block_n;        /* keys per K/V tile                                          */
  int waves;          /* wavefronts per workgroup                                   */
  int num_q_tiles;    /* ceil(Nq / block_m)                                         */
  int64_t grid;       /* workgroups launched = B * (Hq / heads_per_wg) * num_q_tiles */
  int lds_bytes;      /* LDS per workgroup                                          */
  int64_t kv_tiles;   /* K/V tiles visited, summed over all workgroups              */
  int heads_per_wg;   /* query heads per workgroup (sharing a K/V head), block_m rows each */
} fa_plan_info;

/*
 * fa_fwd_plan — the plan fa_fwd would launch for these sizes and options, computed on the host.
 * Same validation rules as fa_fwd for the arguments it takes. Returns FA_OK and fills *info.
 */
fa_status fa_fwd_plan(int B, int Nq, int Nk, int Hq, int Hkv, int D, int causal, int window_left,
                      int window_right, fa_dtype dtype, fa_plan_info* info);

/*
 * fa_kv_tile_range — for query rows [row_begin, row_end) the K/V tiles of `block_n` keys that
 * hold at least one admitted key lie in [*tile_begin, *tile_end) (empty when equal). For the
 * rows [row_begin, row_end) and tile t, *full / *partial / *skipped (each may be NULL) count the
 * tiles in that range that are admitted for every pair, for some pairs, and for none. Host only.
 */
fa_status fa_kv_tile_range(int Nq, int Nk, int causal, int window_left, int window_right,
                           int block_n, int row_begin, int row_end, int* tile_begin, int* tile_end,
                           int* full, int* partial, int* skipped);

/*
 * fa_block_order — for each workgroup id 0 .. n-1 of a forward launch of n = batches * heads *
 * num_tiles workgroups, the (batch, head, query tile) it computes: the order in which the
 * kernels visit their work, which decides which XCD (id % 8) and which L2 reads a head's K/V and
 * when. Host only, no device call. heads: query heads per batch; group: query heads per K/V
 * head; causal: nonzero for a causal launch; packed: nonzero for a fa_fwd_varlen launch. b, h, t:
 * host arrays of n ints, written. Returns FA_ERR_NULL for a null array, FA_ERR_SHAPE unless
 * n, num_tiles, heads and group are >= 1, heads % group == 0, n % (heads * num_tiles) == 0 and
 * n < 2^31.
 */
fa_status fa_block_order(int64_t n, int num_tiles, int heads, int group, int causal, int packed, int* b, int* h,
                         int* t);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
