// topk.hip -- per-query top-index_topk selection on gfx950.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 2:
// for each query the indexer keeps the index_topk best-scored tokens.  A query
// at position p has p + 1 candidates; with no more than K of them all are kept.
//
// One 1024-thread workgroup per query row.  Scores become order-preserving
// uint32 keys (held in LDS when the row fits, else re-read from L2), the K-th
// largest key is found by radix select (12 + 12 + 8 bit digits, histograms in
// LDS), and the selection is written by an ordered compaction: each wave owns a
// contiguous segment, counts its "greater" and "equal" keys, and after a scan of
// the 16 segment counts writes positions in ascending order.  Among keys equal
// to the threshold the smallest positions win, so the selected set is exactly
// "score descending, position ascending" and the output is deterministic.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkStageMax = 32768;  // longest row held in LDS (128 KiB of keys)
constexpr int kHistBins = 4096;

struct TopkShared {
    uint32_t keys[kTopkStageMax];
    uint32_t hist[kHistBins];
    int cnt_gt[kTopkWaves];
    int cnt_eq[kTopkWaves];
    int base_eq[kTopkWaves];
    int base_sel[kTopkWaves];
    uint32_t sel_digit;
    int sel_above;
};

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a)
{
    __shared__ TopkShared sh;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int b = blockIdx.x / a.t_count;
    const int t = a.t_begin + blockIdx.x % a.t_count;
    const int L = min(a.kv_len[b], a.Lmax);
    const int n = max(0, min(a.Lmax, L - a.T + t + 1));  // candidates 0 .. p
    const int K = a.K;
    int32_t* dst = a.idx + ((size_t)b * a.T + t) * K;

    if (n <= K) {
        for (int j = tid; j < K; j += kTopkThreads) dst[j] = j < n ? j : -1;
        return;
    }

    const float* src = a.scores + b * a.ld_b + (long long)(t - a.t_begin) * a.ld_t;
    const bool staged = n <= kTopkStageMax;
    if (staged)
        for (int i = tid; i < n; i += kTopkThreads) sh.keys[i] = float_key(src[i]);
    auto key_at = [&](int i) -> uint32_t { return staged ? sh.keys[i] : float_key(src[i]); };

    // ---- radix select of the K-th largest key
    uint32_t prefix = 0, pmask = 0;
    int krem = K;  // how many still to take among keys matching the prefix
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
        const int nbins = pass == 2 ? 256 : 4096;
        for (int i = tid; i < nbins; i += kTopkThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t k = key_at(i);
            if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l sums bins [l*per, (l+1)*per); suffix-scan the lane sums from the top
            const int per = nbins / 64;
            uint32_t s = 0;
            for (int j = 0; j < per; ++j) s += sh.hist[lane * per + j];
            uint32_t incl = s;  // inclusive suffix sum over lanes >= lane
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_down(incl, off, 64);
                if (lane + off < 64) incl += o;
            }
            const uint32_t excl = incl - s;  // lanes strictly above
            const bool here = excl < (uint32_t)krem && incl >= (uint32_t)krem;
            if (here) {
                uint32_t above = excl;
                for (int j = per - 1; j >= 0; --j) {
                    const uint32_t h = sh.hist[lane * per + j];
                    if (above + h >= (uint32_t)krem) {
                        sh.sel_digit = (uint32_t)(lane * per + j);
                        sh.sel_above = (int)above;
                        break;
                    }
                    above += h;
                }
            }
        }
        __syncthreads();
        const uint32_t d = sh.sel_digit;
        krem -= sh.sel_above;
        prefix |= d << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        __syncthreads();
    }
    const uint32_t tau = prefix;  // key of the K-th largest score; take krem keys equal to it

    // ---- ordered compaction over 16 contiguous wave segments
    const int seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int s0 = min(n, wave * seg), s1 = min(n, s0 + seg);
    int gt = 0, eq = 0;
    for (int i0 = s0; i0 < s1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t k = i < s1 ? key_at(i) : 0u;
        gt += __popcll(__ballot(i < s1 && k > tau));
        eq += __popcll(__ballot(i < s1 && k == tau));
    }
    if (lane == 0) {
        sh.cnt_gt[wave] = gt;
        sh.cnt_eq[wave] = eq;
    }
    __syncthreads();
    if (tid == 0) {
        int be = 0, bs = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            sh.base_eq[w] = be;
            sh.base_sel[w] = bs;
            const int take = max(0, min(krem - be, sh.cnt_eq[w]));
            bs += sh.cnt_gt[w] + take;
            be += sh.cnt_eq[w];
        }
    }
    __syncthreads();
    int run_eq = sh.base_eq[wave], run_sel = sh.base_sel[wave];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i0 = s0; i0 < s1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t k = i < s1 ? key_at(i) : 0u;
        const bool is_gt = i < s1 && k > tau;
        const bool is_eq = i < s1 && k == tau;
        const uint64_t meq = __ballot(is_eq);
        const int eq_rank = run_eq + __popcll(meq & below);
        const bool sel = is_gt || (is_eq && eq_rank < krem);
        const uint64_t msel = __ballot(sel);
        if (sel) dst[run_sel + __popcll(msel & below)] = i;
        run_eq += __popcll(meq);
        run_sel += __popcll(msel);
    }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    topk_kernel<<<dim3(a.B * a.t_count), kTopkThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
