// dsa_kernels.h -- internal launch interface between the C ABI layer and the
// gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Lightning-indexer scores for queries [t_begin, t_begin + t_count) of every
// sequence.  Output row of (b, t) starts at scores + b * ld_b + (t - t_begin) * ld_t.
struct IndexerArgs {
    int B, T, Lmax, H, D;
    int t_begin, t_count;
    const void* q;          // [B,T,H,D] (rows of the full query tensor)
    const float* q_scale;   // [B,T,H] fp8 only
    const float* w;         // [B,T,H]
    const void* k;          // [B,Lmax,D]
    const float* k_scale;   // [B,Lmax] fp8 only
    const int32_t* kv_len;  // [B]
    float* scores;
    long long ld_b, ld_t;
    int fill;               // write -inf for every s > p(t)
    uint32_t* zero;         // optional: words [0, zero_words) are cleared by the launch
    long long zero_words;   //   (a following top-k's counters, see topk_zero_words)
    // optional (decode tiling, t_count <= 2): the split top-k's row histograms
    // (topk_split_hist), already zero, receive the counts of the scores written:
    // per row r = b * t_count + (t - t_begin), hist[r * 4096 + (key >> 20)] and
    // coarse[r * 64 + (key >> 26)] for key = float_key(score) of positions 0 .. p(t)
    uint32_t* hist;
    uint32_t* coarse;
    // streaming top-k (launch_index_topk): per chunk row a list of sel_cap
    // (key, position) pairs in place of the score row; the top sel_k positions of
    // row (b, t) go to sel_idx[(b * T + t) * sel_k ..]
    uint32_t* sel_cand;     // [B * t_count, sel_cap, 2]
    int sel_cap, sel_k;
    int32_t* sel_idx;
};

// Top-k over score rows laid out as in IndexerArgs; writes idx rows of the full
// [B,T,K] tensor for queries [t_begin, t_begin + t_count).
struct TopkArgs {
    int B, T, Lmax, K;
    int t_begin, t_count;
    const float* scores;
    long long ld_b, ld_t;
    const int32_t* kv_len;
    int32_t* idx;
    void* ws;               // topk_workspace_bytes(B, t_count, Lmax, K) bytes, 16-byte aligned
    int pre_zeroed;         // the first topk_zero_words(*this) words of ws are already zero
    int hist_done;          // split path: the row histograms were built with the scores
};

// Sparse absorbed MLA for queries [t_begin, t_begin + t_count).
struct MlaArgs {
    int B, T, Lmax, H, Dqk, Dv, K;
    int t_begin, t_count;
    float sm_scale;
    const void* q;          // [B,T,H,Dqk] (e4m3 codes for the fp8 kernel)
    const float* q_scale;   // [B,T,H] row scales of the fp8 codes, else null
    const void* kv;         // [B,Lmax,Dqk] (fp8: [B,Lmax,Dqk + 16] cache rows, codes then scale)
    const int32_t* idx;     // [B,T,K]
    const int32_t* kv_len;  // [B]
    void* out;              // [B,T,H,Dv]
    float* lse;             // [B,T,H] or null
    void* part;             // split partials (workspace) or null
    int n_split;
};

bool indexer_supported(int dtype, int D, int H);
hipError_t launch_indexer(int dtype, const IndexerArgs& a, hipStream_t s);
// Indexer scores and top-k in one pass, without the score matrix (IndexerArgs sel_*).
hipError_t launch_index_topk(int dtype, const IndexerArgs& a, hipStream_t s);
int index_topk_cap(int K);  // list entries per row

// Workspace of one top-k launch over B * t_count rows (0 when none is needed).
size_t topk_workspace_bytes(int B, int t_count, int Lmax, int K);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Words at the start of the workspace that the launch clears first (0 when none);
// a preceding kernel on the same stream may clear them instead (pre_zeroed).
size_t topk_zero_words(const TopkArgs& a);
// The split path's row histograms inside the workspace (null when the launch does
// not take the split path); a launch that fills them sets hist_done.
struct TopkHist {
    uint32_t* hist;    // [B * t_count][4096]
    uint32_t* coarse;  // [B * t_count][64]
};
TopkHist topk_split_hist(const TopkArgs& a);
// Clears the topk_zero_words(a) words at the start of a.ws.
hipError_t launch_topk_zero(const TopkArgs& a, hipStream_t s);

// Sparse MLA backward for queries [t_begin, t_begin + t_count) of every
// sequence.  Chunk rows are r = b * t_count + (t - t_begin); Hp = H rounded up
// to 16 (the padded heads hold zeros).
struct MlaBwdArgs {
    int B, T, Lmax, H, Hp, K, Dqk, Dv;
    int t_begin, t_count, n_split;
    int accumulate;         // dkv holds earlier gradients (else the call cleared it)
    float sm;
    const uint16_t* q;      // [B,T,H,Dqk] bf16
    const uint16_t* kv;     // [B,Lmax,Dqk] bf16
    const int32_t* idx;     // [B,T,K]
    const int32_t* kv_len;  // [B]
    const float* lse;       // [B,T,H] (forward log-sum-exp, natural log)
    const uint16_t* dout;   // [B,T,H,Dv] bf16
    float* dq;              // [B,T,H,Dqk] out
    float* dkv;             // [B,Lmax,Dqk] accumulated into
    float* Dd;              // [rows, n_split, Hp] workspace: per-split sums of p * dP
    uint16_t* qT;           // [rows, Dqk, Hp]    workspace
    uint16_t* dT;           // [rows, Dv, Hp]     workspace
    float* P;               // [rows, K, Hp]      workspace
    float* DP;              // [rows, K, Hp]      workspace
};
bool mla_bwd_supported(int dtype, int Dqk, int Dv, int H);
hipError_t launch_mla_bwd_chunk(const MlaBwdArgs& a, hipStream_t s);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);

bool mla_supported(int dtype, int Dqk, int Dv);
int mla_split_count(int B, int t_count, int H, int K);
size_t mla_partial_bytes(int dtype, int B, int t_count, int H, int Dv, int n_split);
hipError_t launch_mla(int dtype, const MlaArgs& a, hipStream_t s);

// zero / zero_words: optional words that the launch also clears (a following
// top-k's counters).
hipError_t launch_rotate_quant(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, float* scales,
                               hipStream_t s, uint32_t* zero = nullptr, long long zero_words = 0);
// Per-row e4m3 quantisation without rotation (dim a multiple of 16, at most 1024):
// codes at codes + row * cpitch; the scale to scales[row], or with tail into the
// 16 bytes after the codes (fp32 scale, 12 zero bytes).
hipError_t launch_quant_rows(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, int64_t cpitch,
                             float* scales, int tail, hipStream_t s);
// The index queries' rotate + quantise (rows x dim, bf16) and the MLA queries'
// quantisation (mrows x mdim, bf16) in one launch, with the results of the two.
hipError_t launch_fp8_queries(int64_t rows, int dim, const void* x, uint8_t* codes, float* scales, int64_t mrows,
                              int mdim, const void* mx, uint8_t* mcodes, float* mscales, hipStream_t s,
                              uint32_t* zero = nullptr, long long zero_words = 0);
// Rotate + quantise rows [B, t_new, dim] into cache rows kv_len[b] - t_new + t of [B, max_kv, dim].
hipError_t launch_cache_append(int batch, int t_new, int max_kv, int dim, const void* x, int x_dtype,
                               const int32_t* kv_len, uint8_t* codes, float* scales, hipStream_t s);

}  // namespace dsa
