/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention forward path.
 *
 * What it computes (DeepSeek-V3.2 model documentation page, section "DeepSeek
 * Sparse Attention (DSA)"):
 *   1. lightning indexer: an index score between each query and every previous
 *      key of a single-head index-key cache of width index_head_dim (item 1 and
 *      the paragraph on the indexer key cache).  Score form:
 *          I[t,s] = sum_h w[t,h] * relu(q_idx[t,h,:] . k_idx[s,:]);
 *      with an FP8 indexer both operands are e4m3 codes of Hadamard-rotated
 *      vectors with one fp32 scale per row (the rotation is orthogonal, so the
 *      scores are those of the unrotated vectors up to quantisation);
 *   2. fine-grained token selection: each query keeps its top index_topk
 *      tokens (item 2);
 *   3. MLA attention only over the selected tokens (item 2), in absorbed-latent
 *      form: one latent row [c_kv (v_dim) | k_rope] per token is the key of all
 *      heads and its first v_dim columns are the value; the output is the
 *      v_dim-wide latent per head plus its log-sum-exp.
 * Each layer runs its own indexer (the page's note on per-layer indexers): the
 * library keeps no state between calls.
 *
 * Conventions shared by every entry point
 *   - Sequence b holds kv_len[b] tokens (device int32 array); its T queries are
 *     its last T tokens: query t sits at position p(t) = L_b - T + t with
 *     L_b = min(kv_len[b], max_kv), and sees keys s = 0 .. p(t), itself included.
 *     A row with p(t) < 0 sees nothing (scores all -inf, indices all -1,
 *     output 0, lse -inf).  kv_len is not read on the host.
 *   - Tensors are dense, row-major, innermost dimension contiguous, with base
 *     pointers aligned to 16 bytes.  Every pointer except the shape is a device
 *     pointer.  The caller allocates and owns every buffer, the workspace
 *     included; the library allocates nothing and holds no state.
 *   - Every call only enqueues work on `stream` and returns; it never waits.
 *     Argument errors are found on the host before anything is enqueued and
 *     return a negative status with nothing written.  A failed launch returns
 *     DSA_ERR_HIP.  Two calls may share a workspace only if they are ordered.
 *   - bf16 is the 16-bit brain float; fp8 is the OCP E4M3FN format (bias 7,
 *     largest finite 448, no infinities).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_F32 = 0,
    DSA_BF16 = 1,
    DSA_FP8_E4M3 = 2
} dsa_dtype;

typedef enum {
    DSA_OK = 0,
    DSA_ERR_NULL = -1,        /* a required pointer is NULL                         */
    DSA_ERR_SHAPE = -2,       /* a size is <= 0 or inconsistent (e.g. T > max_kv)    */
    DSA_ERR_DTYPE = -3,       /* dtype value or combination not accepted             */
    DSA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                    */
    DSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required             */
    DSA_ERR_UNSUPPORTED = -6, /* valid but not built (a head width, a head count)    */
    DSA_ERR_HIP = -7,         /* the HIP runtime reported an error on launch         */
    DSA_ERR_SCRATCH = -8,     /* dsa_forward_noalloc: needs more than its scratch    */
    /* Not statuses: they give the type the range of int32_t, so that any int a
     * caller passes to dsa_status_string is a valid value of the type. */
    DSA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    DSA_STATUS_RANGE_MAX_ = 2147483647
} dsa_status;

/* Problem description.  Dtype fields hold dsa_dtype values. */
typedef struct {
    int32_t batch;      /* B  sequences                                             */
    int32_t n_q;        /* T  queries per sequence (1 for decode)                   */
    int32_t max_kv;     /* L_max  cache capacity (rows of k_idx / kv per sequence)  */
    int32_t idx_heads;  /* H_I  index_n_heads, 1..64                                */
    int32_t idx_dim;    /* D_I  index_head_dim                                      */
    int32_t topk;       /* K  index_topk, 1..4096                                   */
    int32_t heads;      /* H  MLA query heads, >= 1                                 */
    int32_t qk_dim;     /* D_qk = kv_lora_rank + qk_rope_head_dim (key width)       */
    int32_t v_dim;      /* D_v  = kv_lora_rank (value = first D_v columns of a row) */
    float sm_scale;     /* softmax scale applied to q . k, finite and > 0; no default */
    int32_t idx_dtype;  /* DSA_F32 | DSA_BF16 | DSA_FP8_E4M3                         */
    int32_t mla_dtype;  /* DSA_F32 | DSA_BF16 | DSA_FP8_E4M3                         */
} dsa_shape;

/*
 * Supported sizes (anything else returns DSA_ERR_UNSUPPORTED):
 *   indexer  idx_dtype F32: idx_dim in {32, 64, 128};  BF16 / FP8: idx_dim = 128;
 *            idx_heads 1..64 (padded internally to 16 or 64).
 *   MLA      (mla_dtype, qk_dim, v_dim) in {(F32, 80, 64), (BF16, 576, 512),
 *            (BF16, 192, 128), (FP8_E4M3, 576, 512)}; any heads >= 1.
 *   top-k    topk <= 4096, max_kv <= 1 << 20.
 *   all      batch <= 65535; batch * n_q <= 2^30; with an MLA,
 *            batch * n_q * heads <= 2^30.
 */

/* Lightning-indexer scores.
 *   q_idx  [B,T,H_I,D_I]  idx_dtype (fp8: e4m3 codes, uint8)
 *   q_scale[B,T,H_I] f32  fp8 only: dequantisation scale of each q_idx row (else NULL)
 *   w      [B,T,H_I] f32  per-head weights of the head sum
 *   k_idx  [B,L_max,D_I]  idx_dtype (fp8: codes)
 *   k_scale[B,L_max] f32  fp8 only: scale of each k_idx row (else NULL)
 *   kv_len [B] int32
 *   scores [B,T,L_max] f32 out: I[t,s] for s <= p(t), -inf for every other s.
 * fp8: I[t,s] = k_scale[s] * sum_h w[t,h] q_scale[t,h] relu(code(q_h) . code(k_s)). */
dsa_status dsa_index_scores(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                            const float* w, const void* k_idx, const float* k_scale,
                            const int32_t* kv_len, float* scores, hipStream_t stream);

/* Indexer scores and per-query top-k in one pass, without the [T, L] score
 * matrix (page items 1 and 2 fused; the streaming form for long prefill).  Each
 * query row keeps a list of candidate (score, position) pairs in the workspace:
 * every causal key joins until the list fills, the list is then cut to the
 * row's exact top K and later keys join only when they score above the K-th.
 * The result equals dsa_index_scores followed by dsa_topk on the same inputs,
 * bit for bit.
 *   q_idx, q_scale, w, k_idx, k_scale, kv_len as for dsa_index_scores.
 *   idx [B,T,K] int32 out, as dsa_topk writes it (ascending positions, -1 padded).
 *   workspace (256-byte aligned): dsa_index_topk_workspace_size(shape) bytes run
 *   every query in one pass (B * T * cap * 8 bytes, cap = max(4K, K + 64)
 *   rounded up to 64); any size >= dsa_index_topk_min_workspace_size works, the
 *   queries then running in chunks of ceil(T / 2^k).  Contents are scratch.
 * Errors: as dsa_index_scores and dsa_topk check the shape; NULL pointers ->
 * DSA_ERR_NULL; q_idx or k_idx not 16-byte aligned, w, kv_len, idx or the fp8
 * scales not 4-byte aligned, workspace not 256-byte aligned -> DSA_ERR_ALIGN;
 * workspace NULL or below the minimum -> DSA_ERR_WORKSPACE. */
size_t dsa_index_topk_workspace_size(const dsa_shape* shape);
size_t dsa_index_topk_min_workspace_size(const dsa_shape* shape);
dsa_status dsa_index_topk(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                          const float* w, const void* k_idx, const float* k_scale,
                          const int32_t* kv_len, int32_t* idx, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Per-query top-k (page item 2).
 *   scores [B,T,L_max] f32 (only s <= p(t) is read), kv_len [B] int32
 *   idx    [B,T,K] int32 out: the k_eff = min(K, p(t)+1) positions with the
 *          largest scores, ties broken towards the smaller position, written in
 *          ascending position order, followed by K - k_eff entries of -1.
 *          -0.0 counts as equal to +0.0; NaN scores are not supported.
 *   workspace / ws_bytes: at least dsa_topk_workspace_size(shape) bytes, 16-byte
 *          aligned, owned by the caller; its contents are scratch on entry and exit.
 *          The size is 0 (workspace may be NULL) unless the rows are few and long
 *          (B*T <= 256 and L_max >= 8192), when each row is split over many
 *          workgroups.  Too small: DSA_ERR_WORKSPACE. */
size_t dsa_topk_workspace_size(const dsa_shape* shape);
dsa_status dsa_topk(const dsa_shape* shape, const float* scores, const int32_t* kv_len,
                    int32_t* idx, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Sparse absorbed-latent MLA over given index sets (page item 2).
 *   q   [B,T,H,D_qk]  mla_dtype    kv [B,L_max,D_qk] mla_dtype
 *   idx [B,T,K] int32: entries outside [0, L_b) are skipped; duplicates count twice
 *   out [B,T,H,D_v] mla_dtype out: sum_j softmax_j(z) kv[idx_j, :D_v] with
 *       z_j = sm_scale * q . kv[idx_j]
 *   lse [B,T,H] f32 out (may be NULL): natural-log log-sum-exp of z
 *   A (b,t) with no valid entry gets out = 0 and lse = -inf.
 *   workspace / ws_bytes: at least dsa_sparse_mla_workspace_size(shape) bytes,
 *   16-byte aligned (NULL allowed when the size is 0); scratch on entry and exit.
 * FP8_E4M3 (the page's FP8 precision applied to the latent cache): kv is the
 * fp8 latent cache of dsa_mla_kv_quant_fp8, uint8 [B,L_max,D_qk + 16] (per row the
 * D_qk e4m3 codes, then the row's fp32 scale and 12 zero bytes); q is BF16 and is
 * quantised per (b,t,h) row inside the call with the same codec; out is BF16.
 * The logits are those of the dequantised operands, code * scale; the softmax
 * weights are rounded to bf16 before the value sum. */
size_t dsa_sparse_mla_workspace_size(const dsa_shape* shape);
dsa_status dsa_sparse_mla_fwd(const dsa_shape* shape, const void* q, const void* kv,
                              const int32_t* idx, const int32_t* kv_len, void* out, float* lse,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* Per-row Hadamard rotation + e4m3 quantisation (the FP8 indexer's operand
 * preparation, page item 1):  x' = H x with H the Sylvester Hadamard matrix
 * scaled by 1/sqrt(dim), rounded to fp32; amax = max|x'|; if amax == 0 the codes
 * are 0 and the scale 1, else codes = e4m3_rne(fp32(x' * fp32(448 / amax))) and
 * scale = fp32(amax / 448).
 *   x      [rows, dim]  x_dtype (DSA_F32 or DSA_BF16), dim a power of two, 16..256
 *   codes  [rows, dim]  uint8 out;  scales [rows] f32 out.
 *   x and codes 16-byte aligned (else DSA_ERR_ALIGN), scales 4-byte aligned. */
dsa_status dsa_rotate_quant_fp8(int64_t rows, int32_t dim, const void* x, int32_t x_dtype,
                                uint8_t* codes, float* scales, hipStream_t stream);

/* Index-key cache update for the FP8 indexer (the cache hook that precedes the
 * indexer, page item 1): the t_new newest keys of every sequence are rotated and
 * quantised exactly as by dsa_rotate_quant_fp8 and written into their cache rows.
 *   k_new  [B, t_new, dim] x_dtype (DSA_F32 or DSA_BF16), dim a power of two, 16..256
 *   kv_len [B] int32 (device): sequence lengths that already count the new keys;
 *          key t of sequence b goes to cache row p = kv_len[b] - t_new + t
 *   codes  [B, max_kv, dim] uint8, scales [B, max_kv] f32 (caller-owned cache,
 *          updated in place): rows p of the new keys are overwritten, rows with
 *          p outside [0, max_kv) are skipped, every other row is left as it is.
 * Errors: batch, t_new or max_kv <= 0 -> DSA_ERR_SHAPE; dim not supported ->
 * DSA_ERR_UNSUPPORTED; other x_dtype -> DSA_ERR_DTYPE; NULL pointers -> DSA_ERR_NULL;
 * k_new or codes not 16-byte aligned, kv_len or scales not 4-byte aligned -> DSA_ERR_ALIGN. */
dsa_status dsa_index_cache_append_fp8(int32_t batch, int32_t t_new, int32_t max_kv, int32_t dim,
                                      const void* k_new, int32_t x_dtype, const int32_t* kv_len,
                                      uint8_t* codes, float* scales, hipStream_t stream);

/* Per-row e4m3 quantisation without rotation into fp8 latent-cache rows (the
 * MLA operand of mla_dtype FP8_E4M3): amax = max|x|; if amax == 0 the codes are
 * 0 and the scale 1, else codes = e4m3_rne(fp32(x * fp32(448 / amax))) and
 * scale = fp32(amax / 448) -- the codec of dsa_rotate_quant_fp8 without the
 * rotation, which would mix the value columns with the rope columns.
 *   x       [rows, dim]  x_dtype (DSA_F32 or DSA_BF16), dim a multiple of 16, <= 1024
 *   kv_rows [rows, dim + 16] uint8 out: the dim codes, the fp32 scale, 12 zero bytes.
 *   Rows are independent, so a cache [B, L_max, dim + 16] is filled in one call
 *   and new tokens are appended by pointing kv_rows at their first row.
 * Errors: rows or dim <= 0 -> DSA_ERR_SHAPE; other dims -> DSA_ERR_UNSUPPORTED;
 * other x_dtype -> DSA_ERR_DTYPE; NULL -> DSA_ERR_NULL; x or kv_rows not
 * 16-byte aligned -> DSA_ERR_ALIGN. */
dsa_status dsa_mla_kv_quant_fp8(int64_t rows, int32_t dim, const void* x, int32_t x_dtype,
                                uint8_t* kv_rows, hipStream_t stream);

/* Backward of the sparse MLA (the page calls DSA trainable): for the forward of
 * dsa_sparse_mla_fwd and the gradient dout of its output,
 *   p_j = exp(z_j - lse),  dP_j = dout . v_j,  D = dout . out = sum_j p_j dP_j,
 *   dz_j = p_j (dP_j - D),  dq = sm_scale sum_j dz_j k_j,
 *   dkv[idx_j] += sm_scale dz_j q  (all D_qk columns)  +  p_j dout  (first D_v columns);
 * an index listed twice contributes twice; skipped entries contribute nothing.
 * D is summed from the recomputed p and dP (not read from the rounded output, whose
 * error would dominate dz where the softmax is concentrated), so the forward
 * output itself is not an argument.
 *   mla_dtype BF16 only, (qk_dim, v_dim) in {(576, 512), (192, 128)}, heads 1..128.
 *   q, kv, idx, kv_len as for dsa_sparse_mla_fwd; lse [B,T,H] f32 is that call's
 *   log-sum-exp for the same inputs; dout [B,T,H,D_v] BF16.
 *   dq  [B,T,H,D_qk] f32 out (every row written).
 *   dkv [B,L_max,D_qk] f32: cleared first unless accumulate_dkv != 0, in which
 *       case the gradients are added to what it holds (fp32 atomics: the order of
 *       the additions, and so the last bits, vary from run to run).  When the call
 *       clears dkv, T == 1 and every query's valid entries are strictly increasing
 *       with skipped entries only after them (top-k's layout), each touched word
 *       receives one update and is stored directly: dkv is then bit-reproducible.
 *   workspace (256-byte aligned): dsa_sparse_mla_bwd_workspace_size(shape) bytes
 *   run every query in one pass; any size >= dsa_sparse_mla_bwd_min_workspace_size
 *   works, the queries then being processed in the largest chunk of ceil(T / 2^k)
 *   queries whose buffers fit (per query about K * round_up(H, 16) * 8 bytes of
 *   p and dP plus the transposed q and dout); both size calls return 0 for a shape
 *   this call rejects.
 * Errors: sizes as dsa_sparse_mla_fwd checks them -> DSA_ERR_SHAPE; mla_dtype not
 * BF16 -> DSA_ERR_DTYPE; other (qk_dim, v_dim) or heads -> DSA_ERR_UNSUPPORTED; NULL
 * pointers -> DSA_ERR_NULL; q, kv, dout, dq or dkv not 16-byte aligned, idx, kv_len
 * or lse not 4-byte aligned, workspace not 256-byte aligned -> DSA_ERR_ALIGN;
 * workspace NULL or below the minimum -> DSA_ERR_WORKSPACE; a failed launch ->
 * DSA_ERR_HIP. */
size_t dsa_sparse_mla_bwd_workspace_size(const dsa_shape* shape);
size_t dsa_sparse_mla_bwd_min_workspace_size(const dsa_shape* shape);
dsa_status dsa_sparse_mla_bwd(const dsa_shape* shape, const void* q, const void* kv,
                              const int32_t* idx, const int32_t* kv_len,
                              const float* lse, const void* dout, float* dq, float* dkv,
                              int32_t accumulate_dkv, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* The whole path: (fp8 only) rotate + quantise q_idx, index scores, top-k,
 * (fp8 MLA only) quantise q, sparse MLA.
 *   q_idx  [B,T,H_I,D_I]: idx_dtype for F32/BF16; for FP8 it is the unrotated
 *          BF16 query, rotated and quantised inside the call
 *   w, kv_len, q, kv as above; k_idx / k_scale as in dsa_index_scores (for FP8
 *   the ready e4m3 cache and its row scales, e.g. from dsa_rotate_quant_fp8)
 *   idx_out [B,T,K] int32 out, or NULL to keep the selection in the workspace
 *   out, lse as in dsa_sparse_mla_fwd.
 *   workspace (256-byte aligned): dsa_forward_workspace_size(shape) bytes run
 *   every query in one pass; any size >= dsa_forward_min_workspace_size(shape)
 *   works, the queries then being processed in the largest chunk of
 *   ceil(T / 2^k) queries whose buffers fit.  When not even one query's score
 *   rows fit, each chunk's scores and top-k run fused as in dsa_index_topk
 *   (8 * cap bytes per query row instead of 4 * L_max, cap as there); the
 *   selection, and so out and lse, are the same bit for bit (both paths compute
 *   every score in the same order). */
size_t dsa_forward_workspace_size(const dsa_shape* shape);
size_t dsa_forward_min_workspace_size(const dsa_shape* shape);
dsa_status dsa_forward(const dsa_shape* shape, const void* q_idx, const float* w,
                       const void* k_idx, const float* k_scale, const void* q, const void* kv,
                       const int32_t* kv_len, int32_t* idx_out, void* out, float* lse,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It computes exactly what dsa_forward computes, with
 * the same kernels and the same query chunking, on a workspace that the library
 * holds: one static device array of DSA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU,
 * kept from the library's first use on that GPU until the process ends.  The
 * call itself allocates nothing (no hipMalloc, no allocating library routine);
 * the caller still owns every input and output.
 *   Arguments as for dsa_forward, without workspace / ws_bytes; stream must
 *   belong to the current device (whose scratch is used).
 *   Shapes whose smallest dsa_forward workspace (dsa_forward_min_workspace_size,
 *   or its idx_out == NULL variant) exceeds the scratch are rejected on the host
 *   with DSA_ERR_SCRATCH before anything is enqueued; the DeepSeek-V3.2 decode
 *   shapes (64 x 32K bf16, 16 x 128K fp8) run in one pass, larger prefill in
 *   query chunks.
 *   Every call on one GPU uses that GPU's one scratch array: calls that overlap
 *   on a GPU (concurrent streams, or threads enqueueing at once) race on it and
 *   must be ordered by the caller.  Everything that must start at zero is
 *   cleared by the call's own kernels; the array keeps the last call's contents.
 *   Other errors as for dsa_forward. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status dsa_forward_noalloc(const dsa_shape* shape, const void* q_idx, const float* w,
                               const void* k_idx, const float* k_scale, const void* q, const void* kv,
                               const int32_t* kv_len, int32_t* idx_out, void* out, float* lse,
                               hipStream_t stream);

/* Static text for a status value. */
const char* dsa_status_string(dsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
