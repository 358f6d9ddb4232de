// topk.hip -- per-query top-index_topk selection on gfx950.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 2:
// for each query the indexer keeps the index_topk best-scored tokens.  A query
// at position p has p + 1 candidates; with no more than K of them all are kept.
//
// Every path selects exactly "score descending, position ascending" and writes
// the positions in ascending order.  Scores become order-preserving uint32 keys
// (-0 folded onto +0).
//
// Many rows (prefill): one 1024-thread workgroup per row.  The row's keys sit in
// LDS when they fit (else are re-read from L2); radix select (12 + 12 + 8 bit
// digits, LDS histograms) finds the K-th largest key tau; an ordered compaction
// over 16 contiguous wave segments then writes every key > tau and the first
// (by position) keys == tau.
//
// Few long rows (decode): the row is split over 4096-entry chunks so the whole
// GPU works on it.
//   hist   : each chunk histograms the top 12 bits of its keys in LDS and adds
//            the non-zero bins to the row's global histogram, and its sums over
//            the top 6 bits to the row's 64-bin coarse histogram;
//   filter : each chunk finds the bin d1 holding the K-th largest key (the
//            coarse bin from 64 words, then the fine bin from that bin's 64
//            words), appends keys above d1 to the row's "selected" list and keys
//            in d1 to its "candidate" list (one reservation per workgroup);
//   finish : one workgroup per row resolves the candidates in LDS (radix select
//            on the low 20 bits, then smallest positions among equal keys),
//            merges them with the selected list and sorts the K positions.
// A candidate list that overflows its buffer falls back to the whole-row select.
#include "dsa_common.h"
#include "dsa_kernels.h"

#include <algorithm>

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkStageMax = 32768;  // longest row held in LDS (128 KiB of keys)
constexpr int kHistBins = 4096;
constexpr int kChunk = 4096;          // entries per chunk of the split path
constexpr int kCandCap = 16384;       // candidate buffer per row of the split path
constexpr int kMaxK = 4096;

constexpr int kLocalCand = 2048;  // keys of the threshold bin held for the last two passes

struct TopkShared {
    uint32_t keys[kTopkStageMax];
    uint32_t hist[kHistBins];
    uint32_t cand[kLocalCand];
    int cnt_gt[kTopkWaves];
    int cnt_eq[kTopkWaves];
    int base_eq[kTopkWaves];
    int base_sel[kTopkWaves];
    uint32_t sel_digit;
    int sel_above;
    uint32_t scan_tmp[kTopkWaves];
};

struct FinishShared {
    union {
        struct {
            uint32_t ckey[kCandCap];
            int32_t cidx[kCandCap];
        };
        uint32_t bits[2 * kCandCap];  // position bitmap, reuses the candidate space
    };
    int32_t out[kMaxK];
    uint32_t hist[1024];
    uint32_t sel_digit;
    int sel_above;
    int n_out;
    uint32_t scan_tmp[kTopkWaves];
};

static_assert(2 * kCandCap * 32 >= (1 << 20), "bitmap must cover the longest row");

union TopkUnion {
    TopkShared full;
    FinishShared fin;
};

// Block-wide versions (all NT threads call them; they end with a barrier, after
// which every thread may read *digit and *count): thread t owns bins
// [t*per, (t+1)*per), the per-thread sums are scanned across waves through
// tmp (NT/64 words of LDS), and the one thread whose range holds the k-th
// element walks its bins.
template <int NT>
__device__ __forceinline__ void block_find_desc(const uint32_t* hist, int nbins, uint32_t k, uint32_t* tmp,
                                                uint32_t* digit, int* above_out)
{
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int per = nbins >= NT ? nbins / NT : 1;
    const int b0 = tid * per;
    uint32_t s = 0;
    if (b0 < nbins)
        for (int j = 0; j < per; ++j) s += hist[b0 + j];
    uint32_t incl = s;  // suffix sum over this wave's lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
    }
    if (lane == 0) tmp[wave] = incl;
    __syncthreads();
    for (int v = wave + 1; v < NW; ++v) incl += tmp[v];
    const uint32_t excl = incl - s;
    if (excl < k && incl >= k) {
        uint32_t above = excl;
        for (int j = per - 1; j >= 0; --j) {
            const uint32_t h = hist[b0 + j];
            if (above + h >= k) {
                *digit = (uint32_t)(b0 + j);
                *above_out = (int)above;
                break;
            }
            above += h;
        }
    }
    __syncthreads();
}

template <int NT>
__device__ __forceinline__ void block_find_asc(const uint32_t* hist, int nbins, uint32_t k, uint32_t* tmp,
                                               uint32_t* digit, int* below_out)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int per = nbins >= NT ? nbins / NT : 1;
    const int b0 = tid * per;
    uint32_t s = 0;
    if (b0 < nbins)
        for (int j = 0; j < per; ++j) s += hist[b0 + j];
    uint32_t incl = s;  // prefix sum over this wave's lanes <= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    for (int v = 0; v < wave; ++v) incl += tmp[v];
    const uint32_t excl = incl - s;
    if (excl < k && incl >= k) {
        uint32_t below = excl;
        for (int j = 0; j < per; ++j) {
            const uint32_t h = hist[b0 + j];
            if (below + h >= k) {
                *digit = (uint32_t)(b0 + j);
                *below_out = (int)below;
                break;
            }
            below += h;
        }
    }
    __syncthreads();
}

// Key i of the row: from LDS when the row is staged there, else from memory.
template <bool STAGED> struct RowKeys;
template <> struct RowKeys<true> {
    const uint32_t* keys;
    __device__ __forceinline__ uint32_t operator()(int i) const { return keys[i]; }
};
template <> struct RowKeys<false> {
    const float* src;
    __device__ __forceinline__ uint32_t operator()(int i) const { return float_key(src[i]); }
};

// Whole-row select by one 1024-thread workgroup (n > K): radix select of the
// K-th largest key, then an ordered compaction writing ascending positions.
// Keys are read in batches of kBatch per thread (loads first, then use), so a
// thread has kBatch reads in flight instead of waiting on each one; reads past
// the end are clamped to the last key and ignored.
constexpr int kBatch = 8;

// Radix passes 1 and 2 (key bits 8..19, then 0..7) over keys key_at(0 .. n - 1),
// counting only keys that match the prefix found so far.
template <class KeyAt>
__device__ __forceinline__ void radix_tail(TopkShared& sh, KeyAt key_at, int n, uint32_t& prefix, uint32_t& pmask,
                                           int& krem)
{
    const int tid = threadIdx.x;
#pragma unroll 1
    for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 8 : 0;
        const int nbins = pass == 2 ? 256 : 4096;
        for (int i = tid; i < nbins; i += kTopkThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int base = 0; base < n; base += kTopkThreads * kBatch) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) kk[u] = key_at(min(base + u * kTopkThreads + tid, n - 1));
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (base + u * kTopkThreads + tid < n && (kk[u] & pmask) == prefix)
                    atomicAdd(&sh.hist[(kk[u] >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        block_find_desc<kTopkThreads>(sh.hist, nbins, (uint32_t)krem, sh.scan_tmp, &sh.sel_digit, &sh.sel_above);
        krem -= sh.sel_above;
        prefix |= sh.sel_digit << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        __syncthreads();
    }
}

// Stages a row of n <= PER * 1024 keys in LDS with the histogram of their top 12 bits: all
// of a thread's loads are issued before the first is used (reads past the row are clamped
// to its last key and ignored).
template <int PER>
__device__ __forceinline__ void stage_keys(TopkShared& sh, const float* src, int n)
{
    const int tid = threadIdx.x;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = src[min(u * kTopkThreads + tid, n - 1)];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = u * kTopkThreads + tid;
        if (i < n) {
            const uint32_t k = float_key(v[u]);
            sh.keys[i] = k;
            atomicAdd(&sh.hist[k >> 20], 1u);
        }
    }
}

template <bool STAGED>
__device__ void block_select_impl(TopkShared& sh, const float* src, int n, int K, int32_t* dst)
{
    // keys per thread and batch: reads from LDS need fewer in flight than reads from memory
    constexpr int kBatch = STAGED ? 4 : ::dsa::kBatch;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    // pass 0 (top 12 key bits) runs on the keys as they are loaded (and staged)
    for (int i = tid; i < kHistBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    if constexpr (STAGED) {
        if (n <= 4 * kTopkThreads)
            stage_keys<4>(sh, src, n);
        else if (n <= 8 * kTopkThreads)
            stage_keys<8>(sh, src, n);
        else if (n <= 16 * kTopkThreads)
            stage_keys<16>(sh, src, n);
        else
            stage_keys<kTopkStageMax / kTopkThreads>(sh, src, n);
    } else {
        for (int base = 0; base < n; base += kTopkThreads * kBatch) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) v[u] = src[min(base + u * kTopkThreads + tid, n - 1)];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (base + u * kTopkThreads + tid < n) atomicAdd(&sh.hist[float_key(v[u]) >> 20], 1u);
        }
    }
    __syncthreads();
    block_find_desc<kTopkThreads>(sh.hist, kHistBins, (uint32_t)K, sh.scan_tmp, &sh.sel_digit, &sh.sel_above);
    int krem = K - sh.sel_above;  // how many still to take among keys matching the prefix
    uint32_t prefix = sh.sel_digit << 20, pmask = 0xFFF00000u;
    const int c0 = (int)sh.hist[sh.sel_digit];  // keys in the threshold bin
    RowKeys<STAGED> key_at;
    if constexpr (STAGED)
        key_at.keys = sh.keys;
    else
        key_at.src = src;

    // output segments: wave w writes the selected positions of [w * seg, (w + 1) * seg)
    const int seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int s0 = min(n, wave * seg), s1 = min(n, s0 + seg);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t tau;  // key of the K-th largest score; take krem keys equal to it
    if (c0 <= kLocalCand) {
        // The threshold bin's keys and positions are gathered (positions go to hist[256 ..],
        // which the remaining passes leave alone), each wave over its own output segment:
        // one scan counts the segment's keys in the bin and above it, a second writes the
        // bin's keys at the wave's offset (a scan of the counts, no atomics).
        uint32_t* cpos = sh.hist + 256;
        const uint32_t top = prefix | 0x000FFFFFu;  // keys above the threshold bin exceed this
        int gt = 0, nin = 0;
        for (int i0 = s0; i0 < s1; i0 += 64 * kBatch) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) kk[u] = key_at(min(i0 + 64 * u + lane, n - 1));
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int i = i0 + 64 * u + lane;
                nin += __popcll(__ballot(i < s1 && (kk[u] & pmask) == prefix));
                gt += __popcll(__ballot(i < s1 && kk[u] > top));
            }
        }
        __syncthreads();  // (every thread has read the threshold bin's count)
        if (lane == 0) {
            sh.cnt_gt[wave] = gt;
            sh.base_eq[wave] = nin;
        }
        __syncthreads();
        int at = 0;
        for (int v = 0; v < wave; ++v) at += sh.base_eq[v];
        for (int i0 = s0; i0 < s1; i0 += 64 * kBatch) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) kk[u] = key_at(min(i0 + 64 * u + lane, n - 1));
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int i = i0 + 64 * u + lane;
                const bool in = i < s1 && (kk[u] & pmask) == prefix;
                const uint64_t m = __ballot(in);
                if (in) {
                    const int r = at + __popcll(m & below);
                    sh.cand[r] = kk[u];
                    cpos[r] = (uint32_t)i;
                }
                at += __popcll(m);
            }
        }
        if (tid < kTopkWaves) sh.cnt_eq[tid] = 0;
        __syncthreads();
        // key bits 12..19, 6..11, 0..5 over the c0 gathered keys, by wave 0 alone:
        // a wave's LDS operations complete in order, so its passes need no barriers
        if (wave == 0) {
#pragma unroll 1
            for (int pass = 0; pass < 3; ++pass) {
                const int shift = pass == 0 ? 12 : (pass == 1 ? 6 : 0);
                const int nbins = pass == 0 ? 256 : 64;
                const int per = nbins / 64;  // bins per lane: lane l holds [l * per, (l + 1) * per)
                for (int bin = lane; bin < nbins; bin += 64) sh.hist[bin] = 0;
                for (int cb = 0; cb < c0; cb += 64 * kBatch) {
                    uint32_t kk[kBatch];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) kk[u] = sh.cand[min(cb + 64 * u + lane, c0 - 1)];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u)
                        if (cb + 64 * u + lane < c0 && (kk[u] & pmask) == prefix)
                            atomicAdd(&sh.hist[(kk[u] >> shift) & (nbins - 1)], 1u);
                }
                uint32_t hv[4], sum = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hv[j] = j < per ? sh.hist[lane * per + j] : 0u;
                    sum += hv[j];
                }
                uint32_t incl = sum;  // keys in this lane's bins and all higher ones
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = __shfl_down(incl, off, 64);
                    if (lane + off < 64) incl += o;
                }
                const uint32_t excl = incl - sum;
                int digit = 0;
                uint32_t above = excl;
                const bool mine = excl < (uint32_t)krem && incl >= (uint32_t)krem;
                if (mine) {
                    for (int j = per - 1; j >= 0; --j) {
                        if (above + hv[j] >= (uint32_t)krem) {
                            digit = lane * per + j;
                            break;
                        }
                        above += hv[j];
                    }
                }
                const int fl = __ffsll((unsigned long long)__ballot(mine)) - 1;
                digit = __builtin_amdgcn_readlane(digit, fl);
                above = __builtin_amdgcn_readlane(above, fl);
                krem -= (int)above;
                prefix |= (uint32_t)digit << shift;
                pmask |= (uint32_t)(nbins - 1) << shift;
            }
            if (lane == 0) {
                sh.sel_digit = prefix;
                sh.sel_above = krem;
            }
        }
        __syncthreads();
        prefix = sh.sel_digit;
        krem = sh.sel_above;
        tau = prefix;
        for (int c = tid; c < c0; c += kTopkThreads) {
            const uint32_t k = sh.cand[c];
            const int w = (int)cpos[c] / seg;
            if (k > tau)
                atomicAdd(&sh.cnt_gt[w], 1);
            else if (k == tau)
                atomicAdd(&sh.cnt_eq[w], 1);
        }
    } else {
        __syncthreads();  // every thread has read the threshold bin's count
        radix_tail(sh, key_at, n, prefix, pmask, krem);
        tau = prefix;
        int gt = 0, eq = 0;
        for (int i0 = s0; i0 < s1; i0 += 64 * kBatch) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) kk[u] = key_at(min(i0 + 64 * u + lane, n - 1));
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const bool in = i0 + 64 * u + lane < s1;
                gt += __popcll(__ballot(in && kk[u] > tau));
                eq += __popcll(__ballot(in && kk[u] == tau));
            }
        }
        if (lane == 0) {
            sh.cnt_gt[wave] = gt;
            sh.cnt_eq[wave] = eq;
        }
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
    for (int i0 = s0; i0 < s1; i0 += 64 * kBatch) {
        uint32_t kk[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) kk[u] = key_at(min(i0 + 64 * u + lane, n - 1));
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + 64 * u + lane;
            const bool is_gt = i < s1 && kk[u] > tau;
            const bool is_eq = i < s1 && kk[u] == tau;
            const uint64_t meq = __ballot(is_eq);
            const int eq_rank = run_eq + __popcll(meq & below);
            const bool sel = is_gt || (is_eq && eq_rank < krem);
            const uint64_t msel = __ballot(sel);
            if (sel) dst[run_sel + __popcll(msel & below)] = i;
            run_eq += __popcll(meq);
            run_sel += __popcll(msel);
        }
    }
}

__device__ __forceinline__ void block_select(TopkShared& sh, const float* src, int n, int K, int32_t* dst)
{
    if (n <= kTopkStageMax)
        block_select_impl<true>(sh, src, n, K, dst);
    else
        block_select_impl<false>(sh, src, n, K, dst);
}

__device__ __forceinline__ void row_of(const TopkArgs& a, int r, int& b, int& t, int& n)
{
    b = r / a.t_count;
    t = a.t_begin + r % a.t_count;
    const int L = min(a.kv_len[b], a.Lmax);
    n = max(0, min(a.Lmax, L - a.T + t + 1));  // candidates 0 .. p
}

__device__ __forceinline__ const float* row_scores(const TopkArgs& a, int b, int t)
{
    return a.scores + b * a.ld_b + (long long)(t - a.t_begin) * a.ld_t;
}

__device__ __forceinline__ void write_all(int32_t* dst, int n, int K)
{
    for (int j = threadIdx.x; j < K; j += blockDim.x) dst[j] = j < n ? j : -1;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a)
{
    __shared__ TopkShared sh;
    int b, t, n;
    row_of(a, blockIdx.x, b, t, n);
    int32_t* dst = a.idx + ((size_t)b * a.T + t) * a.K;
    if (n <= a.K) {
        write_all(dst, n, a.K);
        return;
    }
    block_select(sh, row_scores(a, b, t), n, a.K, dst);
}

// ------------------------------------------------------------ split path
constexpr int kCoarse = 64;  // coarse bins: the top 6 key bits (64 fine bins each)

struct SplitWs {
    uint32_t* hist;  // [rows][4096]
    uint32_t* coarse;  // [rows][64]
    uint32_t* cnt;   // [rows][4]: selected count, candidate count (one 64-bit word, 8-byte aligned)
    int32_t* sel;    // [rows][K]
    uint2* cand;     // [rows][kCandCap] (key, position)
};

__device__ __forceinline__ SplitWs split_ws(const TopkArgs& a)
{
    const size_t rows = (size_t)a.B * a.t_count;
    char* p = (char*)a.ws;
    SplitWs w;
    w.hist = (uint32_t*)p;
    p += rows * kHistBins * 4;
    w.coarse = (uint32_t*)p;
    p += rows * kCoarse * 4;
    w.cnt = (uint32_t*)p;
    p += rows * 4 * 4;
    w.sel = (int32_t*)p;
    p += rows * (size_t)a.K * 4;
    w.cand = (uint2*)p;
    return w;
}

size_t split_ws_bytes(size_t rows, int K)
{
    return rows * ((kHistBins + kCoarse) * 4 + 16 + (size_t)K * 4 + (size_t)kCandCap * 8);
}

size_t split_zero_words(size_t rows) { return rows * (kHistBins + kCoarse + 4); }

__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a)
{
    __shared__ uint32_t lh[kHistBins];
    int b, t, n;
    row_of(a, blockIdx.y, b, t, n);
    const int c0 = blockIdx.x * kChunk;
    if (n <= a.K || c0 >= n) return;
    const int c1 = min(n, c0 + kChunk);
    const SplitWs w = split_ws(a);
    const float* src = row_scores(a, b, t);
    // all of this thread's keys are loaded before the first histogram update
    constexpr int PER = kChunk / 256;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = src[min(c0 + (int)threadIdx.x + 256 * j, c1 - 1)];
    for (int i = threadIdx.x; i < kHistBins; i += 256) lh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (c0 + (int)threadIdx.x + 256 * j < c1) atomicAdd(&lh[float_key(v[j]) >> 20], 1u);
    __syncthreads();
    uint32_t* gh = w.hist + (size_t)blockIdx.y * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
        const uint32_t v = lh[i];
        if (v) atomicAdd(&gh[i], v);
    }
    // coarse bins: thread t sums fine bins [16t, 16t + 16), four threads per coarse bin
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < kHistBins / 256; ++j) cs += lh[threadIdx.x * (kHistBins / 256) + j];
    cs += __shfl_xor(cs, 1, 64);
    cs += __shfl_xor(cs, 2, 64);
    if ((threadIdx.x & 3) == 0 && cs) atomicAdd(&w.coarse[(size_t)blockIdx.y * kCoarse + threadIdx.x / 4], cs);
}

// Wave-level search over 64 bins held one per lane (bin = lane), from the top:
// the lane whose bin holds the k-th largest element, and the count above it.
__device__ __forceinline__ void wave_find_desc64(uint32_t h, uint32_t k, int& bin, uint32_t& above)
{
    const int lane = lane_id();
    uint32_t incl = h;  // suffix sum over lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
    }
    const uint32_t excl = incl - h;
    const uint64_t hit = __ballot(excl < k && incl >= k);
    bin = hit ? (int)__builtin_ctzll(hit) : 0;
    above = __shfl(excl, bin, 64);
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

constexpr int kFilterPer = kChunk / 256;  // keys per thread in the filter pass

__global__ __launch_bounds__(256) void topk_filter_kernel(TopkArgs a)
{
    __shared__ uint32_t sh_digit;
    __shared__ uint32_t wtot[2][4];
    __shared__ uint32_t gbase[2];
    int b, t, n;
    row_of(a, blockIdx.y, b, t, n);
    const int c0 = blockIdx.x * kChunk;
    if (n <= a.K || c0 >= n) return;
    const int c1 = min(n, c0 + kChunk);
    const SplitWs w = split_ws(a);
    const size_t row = blockIdx.y;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const float* src = row_scores(a, b, t);
    // keys of this thread: c0 + tid + 256 * j, loaded while the threshold is found (reads
    // past the chunk are clamped to its last key and ignored)
    uint32_t key[kFilterPer];
#pragma unroll
    for (int j = 0; j < kFilterPer; ++j)  // the last read of these scores: non-temporal
        key[j] = float_key(__builtin_nontemporal_load(src + min(c0 + tid + 256 * j, c1 - 1)));
    // the bin d1 of the K-th largest key: coarse bin first (64 words), then its 64 fine bins
    if (wave == 0) {
        int cb, fb;
        uint32_t above_c, above_f;
        wave_find_desc64(w.coarse[row * kCoarse + lane], (uint32_t)a.K, cb, above_c);
        wave_find_desc64(w.hist[row * kHistBins + cb * 64 + lane], (uint32_t)a.K - above_c, fb, above_f);
        if (lane == 0) sh_digit = (uint32_t)(cb * 64 + fb);
    }
    __syncthreads();
    const uint32_t d1 = sh_digit;
    uint32_t ns = 0, nc = 0;
#pragma unroll
    for (int j = 0; j < kFilterPer; ++j) {
        const bool ok = c0 + tid + 256 * j < c1;
        const uint32_t dg = key[j] >> 20;
        ns += (ok && dg > d1) ? 1u : 0u;
        nc += (ok && dg == d1) ? 1u : 0u;
    }
    const uint32_t is = wave_incl_scan(ns), ic = wave_incl_scan(nc);
    if (lane == 63) {
        wtot[0][wave] = is;
        wtot[1][wave] = ic;
    }
    __syncthreads();
    if (tid == 0) {  // one reservation per workgroup for both lists: (candidates << 32) + selected
        const uint32_t ts = wtot[0][0] + wtot[0][1] + wtot[0][2] + wtot[0][3];
        const uint32_t tc = wtot[1][0] + wtot[1][1] + wtot[1][2] + wtot[1][3];
        uint64_t old = 0;
        if (ts | tc)
            old = atomicAdd(reinterpret_cast<unsigned long long*>(&w.cnt[row * 4]),
                            ((unsigned long long)tc << 32) | ts);
        gbase[0] = (uint32_t)old;
        gbase[1] = (uint32_t)(old >> 32);
    }
    __syncthreads();
    uint32_t ps = gbase[0] + is - ns, pc = gbase[1] + ic - nc;
    for (int v = 0; v < wave; ++v) {
        ps += wtot[0][v];
        pc += wtot[1][v];
    }
    int32_t* sel = w.sel + row * a.K;
    uint2* cand = w.cand + row * kCandCap;
#pragma unroll
    for (int j = 0; j < kFilterPer; ++j) {
        const int i = c0 + tid + 256 * j;
        const uint32_t dg = key[j] >> 20;
        if (i < c1 && dg > d1) sel[ps++] = i;
        if (i < c1 && dg == d1) {
            if (pc < (uint32_t)kCandCap) cand[pc] = make_uint2(key[j], (uint32_t)i);
            ++pc;
        }
    }
}

// Block-wide exclusive scan (1024 threads); `tmp` holds 16 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int u = 0; u < wave; ++u) base += tmp[u];
    return base + incl - v;
}

// Threshold among the candidates of a row's threshold bin (keys ckey, positions
// cidx, n_cand of them; the top 12 key bits are equal): the krem-th largest low
// 20 bits tau_low (radix select on bits 19..10, then 9..0) and, among candidates
// equal to it, the largest position that is still taken (iota; all of them:
// 0xFFFFFFFF).  A candidate is taken iff its low bits exceed tau_low, or equal it
// at a position <= iota.  Block-wide (every thread calls it); hist is 1024 words.
__device__ __forceinline__ void resolve_candidates(const uint32_t* ckey, const int32_t* cidx, int n_cand, int krem,
                                                   uint32_t* hist, uint32_t* scan_tmp, uint32_t* sel_digit,
                                                   int* sel_above, uint32_t& tau_low, uint32_t& iota)
{
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int need = krem;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        for (int i = tid; i < 1024; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += kTopkThreads) {
            const uint32_t k = ckey[i];
            if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1u);
        }
        __syncthreads();
        block_find_desc<kTopkThreads>(hist, 1024, (uint32_t)need, scan_tmp, sel_digit, sel_above);
        need -= *sel_above;
        prefix |= *sel_digit << shift;
        pmask |= 1023u << shift;
        __syncthreads();
    }
    tau_low = prefix;  // low 20 bits of the threshold key
    const int count_eq = (int)hist[tau_low & 1023u];
    __syncthreads();  // every thread has read the histogram before it is cleared again
    // among keys equal to the threshold, keep the `need` smallest positions
    iota = 0xFFFFFFFFu;
    if (need < count_eq) {
        uint32_t ip = 0, im = 0;
        int k2 = need;
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = pass == 0 ? 10 : 0;
            for (int i = tid; i < 1024; i += kTopkThreads) hist[i] = 0;
            __syncthreads();
            for (int i = tid; i < n_cand; i += kTopkThreads) {
                const uint32_t p = (uint32_t)cidx[i];
                if ((ckey[i] & 0xFFFFFu) == tau_low && (p & im) == ip) atomicAdd(&hist[(p >> shift) & 1023u], 1u);
            }
            __syncthreads();
            block_find_asc<kTopkThreads>(hist, 1024, (uint32_t)k2, scan_tmp, sel_digit, sel_above);
            k2 -= *sel_above;
            ip |= *sel_digit << shift;
            im |= 1023u << shift;
            __syncthreads();
        }
        iota = ip;
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_finish_kernel(TopkArgs a)
{
    __shared__ TopkUnion u;
    int b, t, n;
    row_of(a, blockIdx.x, b, t, n);
    const int K = a.K;
    int32_t* dst = a.idx + ((size_t)b * a.T + t) * K;
    if (n <= K) {
        write_all(dst, n, K);
        return;
    }
    const SplitWs w = split_ws(a);
    const size_t row = blockIdx.x;
    const int n_sel = (int)w.cnt[row * 4 + 0];
    const int n_cand = (int)w.cnt[row * 4 + 1];
    if (n_cand > kCandCap) {  // candidate buffer overflowed: select over the whole row
        block_select(u.full, row_scores(a, b, t), n, K, dst);
        return;
    }
    FinishShared& f = u.fin;
    const int tid = threadIdx.x, wave = tid >> 6;
    const uint2* cand = w.cand + row * kCandCap;
    for (int i = tid; i < n_cand; i += kTopkThreads) {
        const uint2 c = cand[i];
        f.ckey[i] = c.x;
        f.cidx[i] = (int32_t)c.y;
    }
    const int krem = K - n_sel;  // candidates to take, 1 <= krem <= n_cand
    uint32_t tau_low, iota;
    resolve_candidates(f.ckey, f.cidx, n_cand, krem, f.hist, f.scan_tmp, &f.sel_digit, &f.sel_above, tau_low, iota);
    // the chosen candidates go to `out` before the bitmap reuses the candidate space
    if (tid == 0) f.n_out = 0;
    __syncthreads();
    for (int i = tid; i < n_cand; i += kTopkThreads) {
        const uint32_t lk = f.ckey[i] & 0xFFFFFu;
        if (lk > tau_low || (lk == tau_low && (uint32_t)f.cidx[i] <= iota)) {
            const int slot = atomicAdd(&f.n_out, 1);
            if (slot < K) f.out[slot] = f.cidx[i];
        }
    }
    __syncthreads();
    const int n_chosen = min(f.n_out, K);
    // bitmap over positions [0, n): set the selected and chosen positions
    uint32_t* bits = f.bits;
    const int n_words = (n + 31) >> 5;
    for (int i = tid; i < n_words; i += kTopkThreads) bits[i] = 0u;
    __syncthreads();
    const int32_t* sel = w.sel + row * K;
    for (int i = tid; i < n_sel; i += kTopkThreads) {
        const int p = sel[i];
        atomicOr(&bits[p >> 5], 1u << (p & 31));
    }
    for (int i = tid; i < n_chosen; i += kTopkThreads) {
        const int p = f.out[i];
        atomicOr(&bits[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // ordered emission: each thread owns a contiguous run of words
    const int per = (n_words + kTopkThreads - 1) / kTopkThreads;
    const int w0 = min(n_words, tid * per), w1 = min(n_words, w0 + per);
    uint32_t cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(bits[i]);
    uint32_t pos = block_excl_scan(cnt, f.hist);
    for (int i = w0; i < w1; ++i) {
        uint32_t m = bits[i];
        while (m) {
            const int bit = __ffs(m) - 1;
            m &= m - 1;
            if (pos < (uint32_t)K) dst[pos] = (i << 5) + bit;
            ++pos;
        }
    }
}

bool use_split(const TopkArgs& a) { return (long long)a.B * a.t_count <= 256 && a.Lmax >= 2 * kChunk; }

}  // namespace

size_t topk_workspace_bytes(int B, int T, int Lmax, int K)
{
    TopkArgs a{};
    a.B = B;
    a.t_count = T;
    a.Lmax = Lmax;
    a.K = K;
    return use_split(a) ? split_ws_bytes((size_t)B * T, K) : 0;
}

size_t topk_zero_words(const TopkArgs& a)
{
    return (a.t_count > 0 && a.B > 0 && use_split(a)) ? split_zero_words((size_t)a.B * a.t_count) : 0;
}

TopkHist topk_split_hist(const TopkArgs& a)
{
    if (topk_zero_words(a) == 0) return TopkHist{nullptr, nullptr};
    const size_t rows = (size_t)a.B * a.t_count;
    uint32_t* p = (uint32_t*)a.ws;  // the layout of split_ws
    return TopkHist{p, p + rows * kHistBins};
}

hipError_t launch_topk_zero(const TopkArgs& a, hipStream_t s)
{
    const size_t zw = topk_zero_words(a);
    if (zw == 0) return hipSuccess;
    topk_zero_kernel<<<dim3((unsigned)std::min<size_t>((zw + 255) / 256, 1024)), 256, 0, s>>>((uint32_t*)a.ws, zw);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    const int rows = a.B * a.t_count;
    if (!use_split(a)) {
        topk_kernel<<<dim3(rows), kTopkThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    const size_t zw = split_zero_words(rows);
    if (!a.pre_zeroed)
        topk_zero_kernel<<<dim3((unsigned)std::min<size_t>((zw + 255) / 256, 1024)), 256, 0, s>>>((uint32_t*)a.ws, zw);
    const dim3 grid((a.Lmax + kChunk - 1) / kChunk, rows);
    if (!a.hist_done) topk_hist_kernel<<<grid, 256, 0, s>>>(a);
    topk_filter_kernel<<<grid, 256, 0, s>>>(a);
    topk_finish_kernel<<<dim3(rows), kTopkThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
