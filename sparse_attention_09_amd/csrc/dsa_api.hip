// dsa_api.hip -- C ABI of the DSA forward path (declared in include/dsa.h).
//
// Host side only: argument validation (before anything is enqueued), workspace
// carving, query chunking for long prefill and the launch sequence of the
// gfx950 kernels.  Nothing here computes any step of the method.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "dsa.h"
#include "dsa_kernels.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxTopk = 4096;
constexpr int kMaxMlaSplit = 16;  // most list splits of one query (mla_split_count)
constexpr int kMaxKv = 1 << 20;
// Launch-size limits: batch is a grid dimension (at most 65535); query rows
// B * T and query-head rows B * T * H stay below 2^30, so every launch size and
// every row or unit index the kernels form fits an int.
constexpr int kMaxBatch = 65535;
constexpr int64_t kMaxRows = int64_t{1} << 30;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

dsa_status check_common(const dsa_shape* s)
{
    if (!s) return DSA_ERR_NULL;
    if (s->batch <= 0 || s->n_q <= 0 || s->max_kv <= 0) return DSA_ERR_SHAPE;
    if (s->n_q > s->max_kv) return DSA_ERR_SHAPE;
    if (s->max_kv > kMaxKv) return DSA_ERR_UNSUPPORTED;
    if (s->batch > kMaxBatch || (int64_t)s->batch * s->n_q > kMaxRows) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status check_indexer_shape(const dsa_shape* s)
{
    if (s->idx_heads <= 0 || s->idx_dim <= 0) return DSA_ERR_SHAPE;
    if (s->idx_dtype != DSA_F32 && s->idx_dtype != DSA_BF16 && s->idx_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
    if (!dsa::indexer_supported(s->idx_dtype, s->idx_dim, s->idx_heads)) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status check_topk_shape(const dsa_shape* s)
{
    if (s->topk <= 0) return DSA_ERR_SHAPE;
    if (s->topk > kMaxTopk) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status check_mla_shape(const dsa_shape* s)
{
    if (s->heads <= 0 || s->qk_dim <= 0 || s->v_dim <= 0 || s->topk <= 0) return DSA_ERR_SHAPE;
    if (s->v_dim > s->qk_dim) return DSA_ERR_SHAPE;
    if (!isfinite(s->sm_scale) || !(s->sm_scale > 0.f)) return DSA_ERR_SHAPE;
    if (s->mla_dtype != DSA_F32 && s->mla_dtype != DSA_BF16 && s->mla_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
    if (s->topk > kMaxTopk) return DSA_ERR_UNSUPPORTED;
    if (!dsa::mla_supported(s->mla_dtype, s->qk_dim, s->v_dim)) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)s->batch * s->n_q * s->heads > kMaxRows) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status ptr_ok(const void* p, size_t align)
{
    if (!p) return DSA_ERR_NULL;
    if (!aligned(p, align)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

#define DSA_TRY(x)                        \
    do {                                  \
        dsa_status st_ = (x);             \
        if (st_ != DSA_OK) return st_;    \
    } while (0)

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

dsa::IndexerArgs indexer_args(const dsa_shape* s, const void* q, const float* qs, const float* w, const void* k,
                              const float* ks, const int32_t* kv_len, float* scores, int t_begin, int t_count,
                              int fill)
{
    dsa::IndexerArgs a{};
    a.B = s->batch;
    a.T = s->n_q;
    a.Lmax = s->max_kv;
    a.H = s->idx_heads;
    a.D = s->idx_dim;
    a.t_begin = t_begin;
    a.t_count = t_count;
    a.q = q;
    a.q_scale = qs;
    a.w = w;
    a.k = k;
    a.k_scale = ks;
    a.kv_len = kv_len;
    a.scores = scores;
    a.ld_t = s->max_kv;
    a.ld_b = (long long)t_count * s->max_kv;
    a.fill = fill;
    a.zero = nullptr;
    a.zero_words = 0;
    a.hist = nullptr;
    a.coarse = nullptr;
    a.sel_cand = nullptr;
    a.sel_cap = 0;
    a.sel_k = 0;
    a.sel_idx = nullptr;
    return a;
}

// Candidate-list bytes of dsa_index_topk for a query chunk of tc rows.
size_t index_topk_bytes(const dsa_shape* s, int tc)
{
    return align_up((size_t)s->batch * tc * dsa::index_topk_cap(s->topk) * sizeof(uint64_t));
}

dsa::TopkArgs topk_args(const dsa_shape* s, const float* scores, const int32_t* kv_len, int32_t* idx, void* ws,
                        int t_begin, int t_count)
{
    dsa::TopkArgs a{};
    a.B = s->batch;
    a.T = s->n_q;
    a.Lmax = s->max_kv;
    a.K = s->topk;
    a.t_begin = t_begin;
    a.t_count = t_count;
    a.scores = scores;
    a.ld_t = s->max_kv;
    a.ld_b = (long long)t_count * s->max_kv;
    a.kv_len = kv_len;
    a.idx = idx;
    a.ws = ws;
    return a;
}

dsa::MlaArgs mla_args(const dsa_shape* s, const void* q, const float* q_scale, const void* kv, const int32_t* idx,
                      const int32_t* kv_len, void* out, float* lse, void* part, int t_begin, int t_count, int n_split)
{
    dsa::MlaArgs a;
    a.B = s->batch;
    a.T = s->n_q;
    a.Lmax = s->max_kv;
    a.H = s->heads;
    a.Dqk = s->qk_dim;
    a.Dv = s->v_dim;
    a.K = s->topk;
    a.t_begin = t_begin;
    a.t_count = t_count;
    a.sm_scale = s->sm_scale;
    a.q = q;
    a.q_scale = q_scale;
    a.kv = kv;
    a.idx = idx;
    a.kv_len = kv_len;
    a.out = out;
    a.lse = lse;
    a.part = part;
    a.n_split = n_split;
    return a;
}

size_t mla_ws(const dsa_shape* s, int t_count)
{
    const int ns = dsa::mla_split_count(s->batch, t_count, s->heads, s->topk);
    return dsa::mla_partial_bytes(s->mla_dtype, s->batch, t_count, s->heads, s->v_dim, ns);
}

// fp8 MLA: bytes of the queries' e4m3 codes and of their row scales (all T queries).
size_t mla_qcode_bytes(const dsa_shape* s) { return align_up((size_t)s->batch * s->n_q * s->heads * s->qk_dim); }
size_t mla_qscale_bytes(const dsa_shape* s) { return align_up((size_t)s->batch * s->n_q * s->heads * sizeof(float)); }

// Workspace of dsa_sparse_mla_fwd: (fp8) query codes and scales, then the split partials.
struct MlaLayout {
    size_t qcodes = 0, qscale = 0, part = 0, total = 0;
};

MlaLayout mla_layout(const dsa_shape* s)
{
    MlaLayout l;
    size_t off = 0;
    if (s->mla_dtype == DSA_FP8_E4M3) {
        l.qcodes = off;
        off += mla_qcode_bytes(s);
        l.qscale = off;
        off += mla_qscale_bytes(s);
    }
    l.part = off;
    l.total = off + mla_ws(s, s->n_q);
    return l;
}

// Quantise the bf16 queries [B,T,H,D_qk] of an fp8 MLA into codes and row scales.
hipError_t quant_mla_queries(const dsa_shape* s, const void* q, uint8_t* codes, float* scales, hipStream_t stream)
{
    const int64_t rows = (int64_t)s->batch * s->n_q * s->heads;
    return dsa::launch_quant_rows(rows, s->qk_dim, q, DSA_BF16, codes, s->qk_dim, scales, 0, stream);
}

// Workspace layout of dsa_forward for a query chunk of tc rows.  The top-k
// scratch and the MLA split partials share one region: on one stream the top-k
// of a chunk has finished before its MLA starts.  With `stream` the chunk's
// index scores and top-k run fused (launch_index_topk): per row a candidate
// list of index_topk_cap(K) 8-byte words takes the place of the L_max-float
// score row, and the top-k needs no scratch of its own.
struct FwdLayout {
    size_t qcodes = 0, qscale = 0, mqcodes = 0, mqscale = 0, idx = 0, scores = 0, cand = 0, part = 0, total = 0;
    bool stream = false;
};

FwdLayout fwd_layout(const dsa_shape* s, int tc, bool own_idx, bool stream = false)
{
    FwdLayout l;
    size_t off = 0;
    const size_t BT = (size_t)s->batch * s->n_q;
    if (s->idx_dtype == DSA_FP8_E4M3) {
        l.qcodes = off;
        off += align_up(BT * s->idx_heads * s->idx_dim);
        l.qscale = off;
        off += align_up(BT * s->idx_heads * sizeof(float));
    }
    if (s->mla_dtype == DSA_FP8_E4M3) {
        l.mqcodes = off;
        off += mla_qcode_bytes(s);
        l.mqscale = off;
        off += mla_qscale_bytes(s);
    }
    if (own_idx) {
        l.idx = off;
        off += align_up(BT * s->topk * sizeof(int32_t));
    }
    l.stream = stream;
    if (stream) {
        l.cand = off;
        off += align_up((size_t)s->batch * tc * dsa::index_topk_cap(s->topk) * sizeof(uint64_t));
    } else {
        l.scores = off;
        off += align_up((size_t)s->batch * tc * s->max_kv * sizeof(float));
    }
    l.part = off;
    const size_t tk = stream ? 0 : dsa::topk_workspace_bytes(s->batch, tc, s->max_kv, s->topk);
    const size_t pw = mla_ws(s, tc);
    off += align_up(tk > pw ? tk : pw);
    l.total = off;
    return l;
}

dsa_status check_forward_shape(const dsa_shape* s)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_indexer_shape(s));
    DSA_TRY(check_topk_shape(s));
    DSA_TRY(check_mla_shape(s));
    return DSA_OK;
}

// Query-chunk candidates: T, ceil(T/2), ceil(T/4), ..., 1.  The workspace of a
// chunk is not monotone in its size (smaller chunks split the index list more),
// so the smallest workspace is the minimum over the candidates.
int next_chunk(int tc) { return tc <= 1 ? 0 : (tc + 1) / 2; }

size_t min_forward_ws(const dsa_shape* s, bool own_idx)
{
    size_t best = (size_t)-1;
    for (int tc = s->n_q; tc > 0; tc = next_chunk(tc))
        for (int st = 0; st < 2; ++st) {
            const size_t w = fwd_layout(s, tc, own_idx, st == 1).total;
            if (w < best) best = w;
        }
    return best;
}

// The layout dsa_forward runs with in ws_bytes, and its query rows per chunk
// (*tc, 0 when nothing fits): the largest chunk of the score-row path, or, when
// not even one query's score rows fit, the largest chunk of the fused streaming
// path (8·cap bytes per row against 4·L_max: long contexts).  Chunking the score
// rows costs next to nothing (prefill_32k in 256 MiB: 27.4 ms against 28.1 ms in
// one pass), while streaming chunks cost more (29.4 ms there), so streaming is
// only the fallback.
FwdLayout choose_forward_layout(const dsa_shape* s, bool own_idx, size_t ws_bytes, int* tc)
{
    int ts = s->n_q;
    while (ts > 0 && fwd_layout(s, ts, own_idx).total > ws_bytes) ts = next_chunk(ts);
    if (ts == 0) {
        int tx = s->n_q;
        while (tx > 0 && fwd_layout(s, tx, own_idx, true).total > ws_bytes) tx = next_chunk(tx);
        if (tx > 0) {
            *tc = tx;
            return fwd_layout(s, tx, own_idx, true);
        }
    }
    *tc = ts;
    return ts > 0 ? fwd_layout(s, ts, own_idx) : FwdLayout{};
}

// Workspace of dsa_sparse_mla_bwd for a query chunk of tc rows.
struct BwdLayout {
    size_t Dd = 0, qT = 0, dT = 0, P = 0, DP = 0, total = 0;
};

int bwd_heads_padded(const dsa_shape* s) { return (s->heads + 15) / 16 * 16; }

BwdLayout bwd_layout(const dsa_shape* s, int tc)
{
    BwdLayout l;
    const size_t rows = (size_t)s->batch * tc, Hp = (size_t)bwd_heads_padded(s);
    size_t off = 0;
    l.Dd = off;
    off += align_up(rows * kMaxMlaSplit * Hp * sizeof(float));
    l.qT = off;
    off += align_up(rows * s->qk_dim * Hp * 2);
    l.dT = off;
    off += align_up(rows * s->v_dim * Hp * 2);
    l.P = off;
    off += align_up(rows * s->topk * Hp * sizeof(float));
    l.DP = off;
    off += align_up(rows * s->topk * Hp * sizeof(float));
    l.total = off;
    return l;
}

dsa_status check_bwd_shape(const dsa_shape* s)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_mla_shape(s));
    if (s->mla_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (!dsa::mla_bwd_supported(s->mla_dtype, s->qk_dim, s->v_dim, s->heads)) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

}  // namespace

DSA_EXPORT const char* dsa_status_string(dsa_status st)
{
    switch (st) {
        case DSA_OK: return "ok";
        case DSA_ERR_NULL: return "a required pointer is NULL";
        case DSA_ERR_SHAPE: return "invalid or inconsistent sizes";
        case DSA_ERR_DTYPE: return "dtype value or combination not accepted";
        case DSA_ERR_ALIGN: return "pointer not aligned";
        case DSA_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA_ERR_UNSUPPORTED: return "sizes valid but not supported by the built kernels";
        case DSA_ERR_HIP: return "HIP runtime error on launch";
        case DSA_ERR_SCRATCH: return "shape needs more than the library's static scratch (dsa_forward_noalloc)";
        default: break;
    }
    return "unknown status";
}

DSA_EXPORT dsa_status dsa_index_scores(const dsa_shape* s, const void* q_idx, const float* q_scale, const float* w,
                                       const void* k_idx, const float* k_scale, const int32_t* kv_len,
                                       float* scores, hipStream_t stream)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_indexer_shape(s));
    DSA_TRY(ptr_ok(q_idx, 16));
    DSA_TRY(ptr_ok(k_idx, 16));
    DSA_TRY(ptr_ok(w, 4));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(scores, 4));
    if (s->idx_dtype == DSA_FP8_E4M3) {
        DSA_TRY(ptr_ok(q_scale, 4));
        DSA_TRY(ptr_ok(k_scale, 4));
    }
    const dsa::IndexerArgs a =
        indexer_args(s, q_idx, q_scale, w, k_idx, k_scale, kv_len, scores, 0, s->n_q, /*fill=*/1);
    return hip_status(dsa::launch_indexer(s->idx_dtype, a, stream));
}

DSA_EXPORT size_t dsa_index_topk_workspace_size(const dsa_shape* s)
{
    if (check_common(s) != DSA_OK || check_indexer_shape(s) != DSA_OK || check_topk_shape(s) != DSA_OK) return 0;
    return index_topk_bytes(s, s->n_q);
}

DSA_EXPORT size_t dsa_index_topk_min_workspace_size(const dsa_shape* s)
{
    if (check_common(s) != DSA_OK || check_indexer_shape(s) != DSA_OK || check_topk_shape(s) != DSA_OK) return 0;
    return index_topk_bytes(s, 1);
}

DSA_EXPORT dsa_status dsa_index_topk(const dsa_shape* s, const void* q_idx, const float* q_scale, const float* w,
                                     const void* k_idx, const float* k_scale, const int32_t* kv_len, int32_t* idx,
                                     void* workspace, size_t ws_bytes, hipStream_t stream)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_indexer_shape(s));
    DSA_TRY(check_topk_shape(s));
    DSA_TRY(ptr_ok(q_idx, 16));
    DSA_TRY(ptr_ok(k_idx, 16));
    DSA_TRY(ptr_ok(w, 4));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(idx, 4));
    if (s->idx_dtype == DSA_FP8_E4M3) {
        DSA_TRY(ptr_ok(q_scale, 4));
        DSA_TRY(ptr_ok(k_scale, 4));
    }
    if (!workspace) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return DSA_ERR_ALIGN;
    int tc = s->n_q;
    while (tc > 0 && index_topk_bytes(s, tc) > ws_bytes) tc = next_chunk(tc);
    if (tc == 0) return DSA_ERR_WORKSPACE;
    for (int t0 = 0; t0 < s->n_q; t0 += tc) {
        const int cnt = (s->n_q - t0) < tc ? (s->n_q - t0) : tc;
        dsa::IndexerArgs a = indexer_args(s, q_idx, q_scale, w, k_idx, k_scale, kv_len, nullptr, t0, cnt, 0);
        a.sel_cand = (uint32_t*)workspace;
        a.sel_cap = dsa::index_topk_cap(s->topk);
        a.sel_k = s->topk;
        a.sel_idx = idx;
        if (dsa::launch_index_topk(s->idx_dtype, a, stream) != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

DSA_EXPORT size_t dsa_topk_workspace_size(const dsa_shape* s)
{
    if (check_common(s) != DSA_OK || check_topk_shape(s) != DSA_OK) return 0;
    return dsa::topk_workspace_bytes(s->batch, s->n_q, s->max_kv, s->topk);
}

DSA_EXPORT dsa_status dsa_topk(const dsa_shape* s, const float* scores, const int32_t* kv_len, int32_t* idx,
                               void* workspace, size_t ws_bytes, hipStream_t stream)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_topk_shape(s));
    DSA_TRY(ptr_ok(scores, 4));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(idx, 4));
    const size_t need = dsa::topk_workspace_bytes(s->batch, s->n_q, s->max_kv, s->topk);
    if (need > 0) {
        if (!workspace || ws_bytes < need) return DSA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return DSA_ERR_ALIGN;
    }
    const dsa::TopkArgs a = topk_args(s, scores, kv_len, idx, need > 0 ? workspace : nullptr, 0, s->n_q);
    return hip_status(dsa::launch_topk(a, stream));
}

DSA_EXPORT size_t dsa_sparse_mla_workspace_size(const dsa_shape* s)
{
    if (check_common(s) != DSA_OK || check_mla_shape(s) != DSA_OK) return 0;
    return mla_layout(s).total;
}

DSA_EXPORT dsa_status dsa_sparse_mla_fwd(const dsa_shape* s, const void* q, const void* kv, const int32_t* idx,
                                         const int32_t* kv_len, void* out, float* lse, void* workspace,
                                         size_t ws_bytes, hipStream_t stream)
{
    DSA_TRY(check_common(s));
    DSA_TRY(check_mla_shape(s));
    DSA_TRY(ptr_ok(q, 16));
    DSA_TRY(ptr_ok(kv, 16));
    DSA_TRY(ptr_ok(idx, 4));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(out, 16));
    if (lse && !aligned(lse, 4)) return DSA_ERR_ALIGN;
    const int ns = dsa::mla_split_count(s->batch, s->n_q, s->heads, s->topk);
    const MlaLayout lay = mla_layout(s);
    if (lay.total > 0) {
        if (!workspace || ws_bytes < lay.total) return DSA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return DSA_ERR_ALIGN;
    }
    char* ws = (char*)workspace;
    const void* qm = q;
    const float* qms = nullptr;
    if (s->mla_dtype == DSA_FP8_E4M3) {
        uint8_t* qc = (uint8_t*)(ws + lay.qcodes);
        float* qs = (float*)(ws + lay.qscale);
        if (quant_mla_queries(s, q, qc, qs, stream) != hipSuccess) return DSA_ERR_HIP;
        qm = qc;
        qms = qs;
    }
    const dsa::MlaArgs a = mla_args(s, qm, qms, kv, idx, kv_len, out, lse, ws ? ws + lay.part : nullptr, 0, s->n_q, ns);
    return hip_status(dsa::launch_mla(s->mla_dtype, a, stream));
}

DSA_EXPORT dsa_status dsa_rotate_quant_fp8(int64_t rows, int32_t dim, const void* x, int32_t x_dtype,
                                           uint8_t* codes, float* scales, hipStream_t stream)
{
    if (rows <= 0 || dim <= 0) return DSA_ERR_SHAPE;
    if (x_dtype != DSA_F32 && x_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dim < 16 || dim > 256 || (dim & (dim - 1)) != 0) return DSA_ERR_UNSUPPORTED;
    DSA_TRY(ptr_ok(x, 16));
    DSA_TRY(ptr_ok(codes, 16));
    DSA_TRY(ptr_ok(scales, 4));
    return hip_status(dsa::launch_rotate_quant(rows, dim, x, x_dtype, codes, scales, stream));
}

DSA_EXPORT dsa_status dsa_index_cache_append_fp8(int32_t batch, int32_t t_new, int32_t max_kv, int32_t dim,
                                                 const void* k_new, int32_t x_dtype, const int32_t* kv_len,
                                                 uint8_t* codes, float* scales, hipStream_t stream)
{
    if (batch <= 0 || t_new <= 0 || max_kv <= 0) return DSA_ERR_SHAPE;
    if (x_dtype != DSA_F32 && x_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dim < 16 || dim > 256 || (dim & (dim - 1)) != 0) return DSA_ERR_UNSUPPORTED;
    DSA_TRY(ptr_ok(k_new, 16));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(codes, 16));
    DSA_TRY(ptr_ok(scales, 4));
    return hip_status(dsa::launch_cache_append(batch, t_new, max_kv, dim, k_new, x_dtype, kv_len, codes, scales,
                                               stream));
}

DSA_EXPORT dsa_status dsa_mla_kv_quant_fp8(int64_t rows, int32_t dim, const void* x, int32_t x_dtype,
                                           uint8_t* kv_rows, hipStream_t stream)
{
    if (rows <= 0 || dim <= 0) return DSA_ERR_SHAPE;
    if (x_dtype != DSA_F32 && x_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (dim % 16 != 0 || dim > 1024) return DSA_ERR_UNSUPPORTED;
    DSA_TRY(ptr_ok(x, 16));
    DSA_TRY(ptr_ok(kv_rows, 16));
    return hip_status(dsa::launch_quant_rows(rows, dim, x, x_dtype, kv_rows, (int64_t)dim + 16, nullptr, 1, stream));
}

DSA_EXPORT size_t dsa_sparse_mla_bwd_workspace_size(const dsa_shape* s)
{
    if (check_bwd_shape(s) != DSA_OK) return 0;
    return bwd_layout(s, s->n_q).total;
}

DSA_EXPORT size_t dsa_sparse_mla_bwd_min_workspace_size(const dsa_shape* s)
{
    if (check_bwd_shape(s) != DSA_OK) return 0;
    return bwd_layout(s, 1).total;
}

DSA_EXPORT dsa_status dsa_sparse_mla_bwd(const dsa_shape* s, const void* q, const void* kv, const int32_t* idx,
                                         const int32_t* kv_len, const float* lse, const void* dout,
                                         float* dq, float* dkv, int32_t accumulate_dkv, void* workspace,
                                         size_t ws_bytes, hipStream_t stream)
{
    DSA_TRY(check_bwd_shape(s));
    DSA_TRY(ptr_ok(q, 16));
    DSA_TRY(ptr_ok(kv, 16));
    DSA_TRY(ptr_ok(idx, 4));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(lse, 4));
    DSA_TRY(ptr_ok(dout, 16));
    DSA_TRY(ptr_ok(dq, 16));
    DSA_TRY(ptr_ok(dkv, 16));
    if (!workspace) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return DSA_ERR_ALIGN;
    int tc = s->n_q;
    while (tc > 0 && bwd_layout(s, tc).total > ws_bytes) tc = next_chunk(tc);
    if (tc == 0) return DSA_ERR_WORKSPACE;
    const BwdLayout lay = bwd_layout(s, tc);
    char* ws = (char*)workspace;
    if (!accumulate_dkv &&
        dsa::launch_zero_f32(dkv, (long long)s->batch * s->max_kv * s->qk_dim, stream) != hipSuccess)
        return DSA_ERR_HIP;
    for (int t0 = 0; t0 < s->n_q; t0 += tc) {
        dsa::MlaBwdArgs a;
        a.B = s->batch;
        a.T = s->n_q;
        a.Lmax = s->max_kv;
        a.H = s->heads;
        a.Hp = bwd_heads_padded(s);
        a.K = s->topk;
        a.Dqk = s->qk_dim;
        a.Dv = s->v_dim;
        a.t_begin = t0;
        a.t_count = (s->n_q - t0) < tc ? (s->n_q - t0) : tc;
        a.n_split = dsa::mla_split_count(s->batch, a.t_count, s->heads, s->topk);
        a.accumulate = accumulate_dkv ? 1 : 0;
        a.sm = s->sm_scale;
        a.q = (const uint16_t*)q;
        a.kv = (const uint16_t*)kv;
        a.idx = idx;
        a.kv_len = kv_len;
        a.lse = lse;
        a.dout = (const uint16_t*)dout;
        a.dq = dq;
        a.dkv = dkv;
        a.Dd = (float*)(ws + lay.Dd);
        a.qT = (uint16_t*)(ws + lay.qT);
        a.dT = (uint16_t*)(ws + lay.dT);
        a.P = (float*)(ws + lay.P);
        a.DP = (float*)(ws + lay.DP);
        if (dsa::launch_mla_bwd_chunk(a, stream) != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

DSA_EXPORT size_t dsa_forward_workspace_size(const dsa_shape* s)
{
    if (check_forward_shape(s) != DSA_OK) return 0;
    return fwd_layout(s, s->n_q, true).total;
}

DSA_EXPORT size_t dsa_forward_min_workspace_size(const dsa_shape* s)
{
    if (check_forward_shape(s) != DSA_OK) return 0;
    return min_forward_ws(s, true);
}

namespace {

// Argument checks of dsa_forward other than the workspace.
dsa_status check_forward_args(const dsa_shape* s, const void* q_idx, const float* w, const void* k_idx,
                              const float* k_scale, const void* q, const void* kv, const int32_t* kv_len,
                              const int32_t* idx_out, const void* out, const float* lse)
{
    DSA_TRY(check_forward_shape(s));
    DSA_TRY(ptr_ok(q_idx, 16));
    DSA_TRY(ptr_ok(w, 4));
    DSA_TRY(ptr_ok(k_idx, 16));
    DSA_TRY(ptr_ok(q, 16));
    DSA_TRY(ptr_ok(kv, 16));
    DSA_TRY(ptr_ok(kv_len, 4));
    DSA_TRY(ptr_ok(out, 16));
    if (s->idx_dtype == DSA_FP8_E4M3) DSA_TRY(ptr_ok(k_scale, 4));
    if (idx_out && !aligned(idx_out, 4)) return DSA_ERR_ALIGN;
    if (lse && !aligned(lse, 4)) return DSA_ERR_ALIGN;
    return DSA_OK;
}

// The top-k counters of a query chunk that a launch before the indexer may clear
// (0 when the chunk's top-k needs none).  A decode chunk (the indexer's decode
// tiling, at most 2 queries) on the split top-k also gets its row histograms
// from the indexer, so its counters must be zero before the indexer starts.
size_t fused_hist_zero_words(const dsa_shape* s, const float* scores, const int32_t* kv_len, int32_t* idx,
                             void* part, int t0, int cnt)
{
    if (cnt > 2) return 0;
    return dsa::topk_zero_words(topk_args(s, scores, kv_len, idx, part, t0, cnt));
}

// One chunk's index scores and top-k through the score rows.  `cleared`: a
// launch before this one cleared the chunk's top-k counters
// (fused_hist_zero_words words at `part`).
hipError_t forward_scores_topk(const dsa_shape* s, const void* qi, const float* qsc, const float* w, const void* k_idx,
                               const float* k_scale, const int32_t* kv_len, float* scores, int32_t* idx, void* part,
                               int t0, int cnt, bool cleared, hipStream_t stream)
{
    dsa::IndexerArgs ia = indexer_args(s, qi, qsc, w, k_idx, k_scale, kv_len, scores, t0, cnt, 0);
    dsa::TopkArgs ta = topk_args(s, scores, kv_len, idx, part, t0, cnt);
    const size_t zw = dsa::topk_zero_words(ta);
    if (zw > 0 && cnt <= 2) {
        // decode: the indexer builds the row histograms as it writes the scores,
        // which saves the top-k its histogram pass over the score rows
        if (!cleared) {
            const hipError_t e = dsa::launch_topk_zero(ta, stream);
            if (e != hipSuccess) return e;
        }
        const dsa::TopkHist th = dsa::topk_split_hist(ta);
        ia.hist = th.hist;
        ia.coarse = th.coarse;
        ta.pre_zeroed = 1;
        ta.hist_done = 1;
    } else if (zw > 0) {
        // the indexer clears the top-k's counters, which saves the top-k a launch
        ia.zero = (uint32_t*)part;
        ia.zero_words = (long long)zw;
        ta.pre_zeroed = 1;
    }
    const hipError_t e = dsa::launch_indexer(s->idx_dtype, ia, stream);
    return e != hipSuccess ? e : dsa::launch_topk(ta, stream);
}

// The launch sequence of dsa_forward on a checked, 256-byte aligned workspace.
dsa_status forward_run(const dsa_shape* s, const void* q_idx, const float* w, const void* k_idx,
                       const float* k_scale, const void* q, const void* kv, const int32_t* kv_len,
                       int32_t* idx_out, void* out, float* lse, void* workspace, size_t ws_bytes,
                       hipStream_t stream)
{
    const bool own_idx = idx_out == nullptr;
    int tc = 0;
    const FwdLayout lay = choose_forward_layout(s, own_idx, ws_bytes, &tc);
    if (tc == 0) return DSA_ERR_WORKSPACE;

    char* ws = (char*)workspace;
    int32_t* idx = own_idx ? (int32_t*)(ws + lay.idx) : idx_out;
    float* scores = (float*)(ws + lay.scores);
    void* part = ws + lay.part;
    const void* qi = q_idx;
    const float* qsc = nullptr;
    const void* qm = q;
    const float* qms = nullptr;
    const bool fp8_idx = s->idx_dtype == DSA_FP8_E4M3, fp8_mla = s->mla_dtype == DSA_FP8_E4M3;
    const int64_t idx_rows = (int64_t)s->batch * s->n_q * s->idx_heads;
    // the fp8 index queries' preparation also clears the first chunk's top-k counters
    // when that chunk's indexer builds the top-k histograms
    const size_t zw0 =
        (fp8_idx && !lay.stream) ? fused_hist_zero_words(s, scores, kv_len, idx, part, 0, tc < s->n_q ? tc : s->n_q) : 0;
    uint32_t* const zp0 = zw0 > 0 ? (uint32_t*)part : nullptr;
    if (fp8_idx && fp8_mla) {  // both query preparations in one launch
        uint8_t* qc = (uint8_t*)(ws + lay.qcodes);
        float* qs = (float*)(ws + lay.qscale);
        uint8_t* mqc = (uint8_t*)(ws + lay.mqcodes);
        float* mqs = (float*)(ws + lay.mqscale);
        const int64_t mla_rows = (int64_t)s->batch * s->n_q * s->heads;
        if (dsa::launch_fp8_queries(idx_rows, s->idx_dim, q_idx, qc, qs, mla_rows, s->qk_dim, q, mqc, mqs, stream, zp0,
                                    (long long)zw0) != hipSuccess)
            return DSA_ERR_HIP;
        qi = qc;
        qsc = qs;
        qm = mqc;
        qms = mqs;
    } else if (fp8_idx) {
        uint8_t* qc = (uint8_t*)(ws + lay.qcodes);
        float* qs = (float*)(ws + lay.qscale);
        if (dsa::launch_rotate_quant(idx_rows, s->idx_dim, q_idx, DSA_BF16, qc, qs, stream, zp0, (long long)zw0) !=
            hipSuccess)
            return DSA_ERR_HIP;
        qi = qc;
        qsc = qs;
    } else if (fp8_mla) {
        uint8_t* qc = (uint8_t*)(ws + lay.mqcodes);
        float* qs = (float*)(ws + lay.mqscale);
        if (quant_mla_queries(s, q, qc, qs, stream) != hipSuccess) return DSA_ERR_HIP;
        qm = qc;
        qms = qs;
    }
    for (int t0 = 0; t0 < s->n_q; t0 += tc) {
        const int cnt = (s->n_q - t0) < tc ? (s->n_q - t0) : tc;
        if (lay.stream) {
            dsa::IndexerArgs ia = indexer_args(s, qi, qsc, w, k_idx, k_scale, kv_len, nullptr, t0, cnt, 0);
            ia.sel_cand = (uint32_t*)(ws + lay.cand);
            ia.sel_cap = dsa::index_topk_cap(s->topk);
            ia.sel_k = s->topk;
            ia.sel_idx = idx;
            if (dsa::launch_index_topk(s->idx_dtype, ia, stream) != hipSuccess) return DSA_ERR_HIP;
        } else {
            if (forward_scores_topk(s, qi, qsc, w, k_idx, k_scale, kv_len, scores, idx, part, t0, cnt,
                                    t0 == 0 && zw0 > 0, stream) != hipSuccess)
                return DSA_ERR_HIP;
        }
        const int ns = dsa::mla_split_count(s->batch, cnt, s->heads, s->topk);
        const dsa::MlaArgs ma = mla_args(s, qm, qms, kv, idx, kv_len, out, lse, part, t0, cnt, ns);
        if (dsa::launch_mla(s->mla_dtype, ma, stream) != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

// ------------------------------------------------------------ static scratch
// The workspace of dsa_forward_noalloc: one file-scope device array, of which
// every GPU that runs the library holds its own copy until the process ends.
// Host code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address of the current GPU's copy comes
// from hipGetSymbolAddress, looked up once per device and kept here.
constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % kAlign == 0, "scratch size");
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (the symbol lookup runs once per
// device, under the lock, with that device current).
dsa_status device_scratch(void** ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSA_ERR_HIP;
        if (!aligned(p, kAlign)) return DSA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

DSA_EXPORT dsa_status dsa_forward(const dsa_shape* s, const void* q_idx, const float* w, const void* k_idx,
                                  const float* k_scale, const void* q, const void* kv, const int32_t* kv_len,
                                  int32_t* idx_out, void* out, float* lse, void* workspace, size_t ws_bytes,
                                  hipStream_t stream)
{
    DSA_TRY(check_forward_args(s, q_idx, w, k_idx, k_scale, q, kv, kv_len, idx_out, out, lse));
    if (!workspace) return DSA_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return DSA_ERR_ALIGN;
    return forward_run(s, q_idx, w, k_idx, k_scale, q, kv, kv_len, idx_out, out, lse, workspace, ws_bytes, stream);
}

DSA_EXPORT dsa_status dsa_forward_noalloc(const dsa_shape* s, const void* q_idx, const float* w, const void* k_idx,
                                          const float* k_scale, const void* q, const void* kv,
                                          const int32_t* kv_len, int32_t* idx_out, void* out, float* lse,
                                          hipStream_t stream)
{
    DSA_TRY(check_forward_args(s, q_idx, w, k_idx, k_scale, q, kv, kv_len, idx_out, out, lse));
    if (min_forward_ws(s, idx_out == nullptr) > kScratchBytes) return DSA_ERR_SCRATCH;
    void* ws = nullptr;
    DSA_TRY(device_scratch(&ws));
    return forward_run(s, q_idx, w, k_idx, k_scale, q, kv, kv_len, idx_out, out, lse, ws, kScratchBytes, stream);
}
