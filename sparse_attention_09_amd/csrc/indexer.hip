// indexer.hip -- lightning-indexer scores on gfx950 MFMA.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 1:
// every query is scored against every previous key of a single-head index-key
// cache (width index_head_dim).  Score form used: I[t,s] = sum_h w[t,h] *
// relu(q[t,h,:] . k[s,:]); with an FP8 indexer the operands are e4m3 codes and
// I[t,s] = k_scale[s] * sum_h (w[t,h] q_scale[t,h]) relu(codes . codes), which
// equals the dequantised product because relu is positively homogeneous.
//
// Contraction on MFMA with heads on the M axis and keys on N, d on K.  In the C
// tile a lane holds one key and several heads, so relu + the weighted head sum
// run in-lane, followed by a sum across lane groups.  Scores stay fp32 from the
// accumulator on.
//
// Two tilings of the same arithmetic, both on 16x16 MFMA tiles with the same
// contraction order, so that every path yields the same scores to the last bit:
//   decode   (few queries, long cache): each wave owns a strip of 16-key tiles
//            and streams them straight from HBM into registers, all loads of a
//            strip issued before any MFMA (HBM-bound, no LDS, no barriers);
//   prefill: 4 waves x 2 query rows share 64-key LDS tiles.
// Prefill blocks are issued longest-row first.  The prefill tiling also runs
// fused with the top-k of item 2 (launch_index_topk): a wave owns its two query
// rows over the whole key range, so it keeps each row's candidates in a list of
// its own instead of writing the score row, and the [T, L] score matrix is never
// formed.  The fused form and the score rows agreeing bit for bit is what makes
// dsa_index_topk select exactly what dsa_index_scores + dsa_topk select.
#include "dsa_common.h"
#include "dsa_kernels.h"

#include <algorithm>

namespace dsa {
namespace {

template <int DT> struct ElemBytes;
template <> struct ElemBytes<kF32> { static constexpr int v = 4; };
template <> struct ElemBytes<kBF16> { static constexpr int v = 2; };
template <> struct ElemBytes<kFP8> { static constexpr int v = 1; };

// A lane's share of one D-wide row: D/4 elements = NCH 16-byte chunks.  The
// 16-lane group g takes chunks g, g + 4, g + 8, ... (byte offset 64 c + 16 g for
// its c-th chunk), so that one load instruction over a 16-row tile reads 64
// contiguous bytes of every row.
template <int DT, int D> struct Share {
    static constexpr int bytes = D * ElemBytes<DT>::v / 4;
    static constexpr int nch = bytes / 16;
    static_assert(bytes % 16 == 0, "row share must be whole 16-byte chunks");
    static __device__ __forceinline__ int off(int g, int c) { return 64 * c + 16 * g; }
};

// acc += A_share . B_share over the chunk mapping of Share::off.
template <int DT, int NCH>
__device__ __forceinline__ f32x4 dot_share(const u32x4 (&a)[NCH], const u32x4 (&b)[NCH], f32x4 acc)
{
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if constexpr (DT == kBF16) {
            acc = mfma_bf16(a[c], b[c], acc);
        } else if constexpr (DT == kFP8) {
            acc = mfma_fp8(u32x2{a[c][0], a[c][1]}, u32x2{b[c][0], b[c][1]}, acc);
            acc = mfma_fp8(u32x2{a[c][2], a[c][3]}, u32x2{b[c][2], b[c][3]}, acc);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = mfma_f32(__uint_as_float(a[c][e]), __uint_as_float(b[c][e]), acc);
        }
    }
    return acc;
}

// Load query rows (A operand) and the weights of the heads whose scores this
// lane holds in the C tile.  Heads beyond H read as zero weight and zero query.
template <int DT, int D, int HT>
__device__ __forceinline__ void load_query(const IndexerArgs& a, int b, int t, bool valid,
                                           u32x4 (&qa)[HT][Share<DT, D>::nch], float (&wv)[HT][4])
{
    constexpr int NCH = Share<DT, D>::nch;
    constexpr int EB = ElemBytes<DT>::v;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const size_t qrow = ((size_t)b * a.T + t) * a.H;
#pragma unroll
    for (int m = 0; m < HT; ++m) {
        const int h = 16 * m + n;
        const bool ok = valid && h < a.H;
        const char* src = (const char*)a.q + ((qrow + (ok ? h : 0)) * D) * EB;
#pragma unroll
        for (int c = 0; c < NCH; ++c) qa[m][c] = ok ? ld16(src + Share<DT, D>::off(g, c)) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 16 * m + 4 * g + i;
            float wt = 0.f;
            if (valid && hh < a.H) {
                wt = a.w[qrow + hh];
                if constexpr (DT == kFP8) wt *= a.q_scale[qrow + hh];
            }
            wv[m][i] = wt;
        }
    }
}

template <int HT>
__device__ __forceinline__ float head_sum(const f32x4 (&acc)[HT], const float (&wv)[HT][4])
{
    float v = 0.f;
#pragma unroll
    for (int m = 0; m < HT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[m][i], fmaxf(acc[m][i], 0.f), v);
    return group4_sum(v);
}

// Clear the optional words a.zero[0, zero_words): a grid-stride loop over the
// whole launch, run before any other work of the block.
__device__ __forceinline__ void clear_words(const IndexerArgs& a)
{
    if (a.zero == nullptr) return;
    const long long nthreads = (long long)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    const long long id =
        (((long long)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (long long i = id; i < a.zero_words; i += nthreads) a.zero[i] = 0u;
}

__device__ __forceinline__ int seq_len(const IndexerArgs& a, int b)
{
    const int L = a.kv_len[b];
    return L < a.Lmax ? L : a.Lmax;
}

// ---------------------------------------------------------------- decode tiling
// A strip is TPW consecutive 16-key tiles.  A key at or past kend (>= 1) reads
// row kend - 1 instead: its score column is never stored, and unconditional
// loads keep the register prefetch free of waits.
// Scores leave a strip four tiles at a time: lane (n, g) stores key n of tile
// 4 j + g, so one store covers 64 consecutive keys.  The fp8 key scales are
// loaded with the strip in that store layout, so no load waits behind it.
// Keys are read once per call, and bf16 and fp8 key loads are marked
// non-temporal (whole decode steps, measured: 32K context, 64 sequences, bf16
// 191.2 -> 183.4 us; 128K context, 16 sequences, fp8 at 3072 waves 120.4 -> 118.5 us).
template <int TPW> struct StripOut { static constexpr int n = (TPW + 3) / 4; };

template <int DT, int D, int TPW>
__device__ __forceinline__ void load_strip(const IndexerArgs& a, int b, int strip, int kend,
                                           u32x4 (&kb)[TPW][Share<DT, D>::nch], float (&ks)[StripOut<TPW>::n])
{
    constexpr int NCH = Share<DT, D>::nch;
    constexpr int EB = ElemBytes<DT>::v;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const char* kbase = (const char*)a.k + (size_t)b * a.Lmax * D * EB;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int key = min((strip * TPW + i) * 16 + n, kend - 1);
        const char* src = kbase + (size_t)key * D * EB;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const void* p = src + Share<DT, D>::off(g, c);
            if constexpr (DT == kBF16 || DT == kFP8)
                kb[i][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            else
                kb[i][c] = ld16(p);
        }
    }
#pragma unroll
    for (int j = 0; j < StripOut<TPW>::n; ++j) {
        const int key = min((strip * TPW + 4 * j + g) * 16 + n, kend - 1);
        if constexpr (DT == kFP8)
            ks[j] = a.k_scale[(size_t)b * a.Lmax + key];
        else
            ks[j] = 1.f;
    }
}

// Row histograms of the split top-k built beside the decode scores: one LDS
// histogram of the top 12 key bits per query row of the workgroup, added to the
// row's global histograms (fine and 64-bin coarse) when the workgroup ends.
constexpr int kIdxHistBins = 4096;

template <int DT, int D, int HT, int QPW, int TPW>
__device__ __forceinline__ void score_strip(const IndexerArgs& a, int b, int strip,
                                            const u32x4 (&kb)[TPW][Share<DT, D>::nch],
                                            const float (&ks)[StripOut<TPW>::n],
                                            const u32x4 (&qa)[QPW][HT][Share<DT, D>::nch],
                                            const float (&wv)[QPW][HT][4], const int (&tq)[QPW],
                                            const int (&pq)[QPW], const bool (&vq)[QPW], int kend,
                                            uint32_t (*lh)[kIdxHistBins])
{
    constexpr int NCH = Share<DT, D>::nch;
    constexpr int NO = StripOut<TPW>::n;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
        float vv[4 * NO];
#pragma unroll
        for (int i = 0; i < 4 * NO; ++i) vv[i] = 0.f;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if ((strip * TPW + i) * 16 >= kend) break;
            f32x4 acc[HT];
#pragma unroll
            for (int m = 0; m < HT; ++m) acc[m] = dot_share<DT, NCH>(qa[q][m], kb[i], f32x4{0, 0, 0, 0});
            vv[i] = head_sum<HT>(acc, wv[q]);
        }
        if (!vq[q]) continue;
        float* row = a.scores + b * a.ld_b + (long long)(tq[q] - a.t_begin) * a.ld_t;
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const float v = g == 0 ? vv[4 * j] : g == 1 ? vv[4 * j + 1] : g == 2 ? vv[4 * j + 2] : vv[4 * j + 3];
            const int tile = (strip * TPW + 4 * j + g) * 16;
            const int key = tile + n;
            if (4 * j + g < TPW && tile < kend && key < a.Lmax) {
                if (key <= pq[q]) {
                    const float sv = v * ks[j];
                    row[key] = sv;
                    if (a.hist) atomicAdd(&lh[q][float_key(sv) >> 20], 1u);
                } else if (a.fill) {
                    row[key] = -INFINITY;
                }
            }
        }
    }
}

// Persistent waves: the W waves of a sequence take strips w, w + W, ...; the
// loads of the next strip are in flight while the current one is scored.
template <int DT, int D, int HT, int QPW, int TPW>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerArgs a)
{
    constexpr int NCH = Share<DT, D>::nch;
    constexpr int SK = TPW * 16;  // keys per strip
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.z;
    __shared__ uint32_t lh[QPW][kIdxHistBins];
    clear_words(a);
    if (a.hist) {
        for (int i = threadIdx.x; i < QPW * kIdxHistBins; i += 256) (&lh[0][0])[i] = 0u;
        __syncthreads();
    }
    const int L = seq_len(a, b);

    int tq[QPW], pq[QPW];
    bool vq[QPW];
    int kend = 0;
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
        tq[q] = a.t_begin + blockIdx.y * QPW + q;
        vq[q] = tq[q] < a.t_begin + a.t_count;
        pq[q] = vq[q] ? L - a.T + tq[q] : -1;
        kend = max(kend, pq[q] + 1);
    }
    kend = min(kend, a.Lmax);

    u32x4 qa[QPW][HT][NCH];
    float wv[QPW][HT][4];
#pragma unroll
    for (int q = 0; q < QPW; ++q) load_query<DT, D, HT>(a, b, vq[q] ? tq[q] : a.t_begin, vq[q], qa[q], wv[q]);

    const int W = gridDim.x * 4;
    const int w0 = blockIdx.x * 4 + wave;
    const int n_load = (kend + SK - 1) / SK;
    u32x4 kA[TPW][NCH], kB[TPW][NCH];
    float sA[StripOut<TPW>::n], sB[StripOut<TPW>::n];
    // Every prefetch is issued unconditionally (past the end a wave re-reads the
    // strip it holds), so the wait before scoring a strip covers that strip only.
    if (w0 < n_load) {
        load_strip<DT, D, TPW>(a, b, w0, kend, kA, sA);
        for (int s0 = w0;; s0 += 2 * W) {
            const int s1 = s0 + W;
            load_strip<DT, D, TPW>(a, b, s1 < n_load ? s1 : s0, kend, kB, sB);
            score_strip<DT, D, HT, QPW, TPW>(a, b, s0, kA, sA, qa, wv, tq, pq, vq, kend, lh);
            if (s1 >= n_load) break;
            const int s2 = s1 + W;
            load_strip<DT, D, TPW>(a, b, s2 < n_load ? s2 : s1, kend, kA, sA);
            score_strip<DT, D, HT, QPW, TPW>(a, b, s1, kB, sB, qa, wv, tq, pq, vq, kend, lh);
            if (s2 >= n_load) break;
        }
    }
    if (a.fill) {  // -inf for every position past the last scored tile
        const int f0 = (kend + 15) & ~15;
        for (int s = f0 + (w0 * 64 + lane); s < a.Lmax; s += W * 64)
#pragma unroll
            for (int q = 0; q < QPW; ++q)
                if (vq[q]) a.scores[b * a.ld_b + (long long)(tq[q] - a.t_begin) * a.ld_t + s] = -INFINITY;
    }
    if (a.hist) {
        // this workgroup's counts join the rows' histograms: the non-zero fine bins,
        // and the coarse bins (thread t sums fine bins [16 t, 16 t + 16), four
        // threads per coarse bin)
        __syncthreads();
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            if (!vq[q]) continue;
            const size_t r = (size_t)b * a.t_count + (tq[q] - a.t_begin);
            uint32_t* gh = a.hist + r * kIdxHistBins;
            for (int i = threadIdx.x; i < kIdxHistBins; i += 256) {
                const uint32_t c = lh[q][i];
                if (c) atomicAdd(&gh[i], c);
            }
            uint32_t cs = 0;
#pragma unroll
            for (int j = 0; j < kIdxHistBins / 256; ++j) cs += lh[q][threadIdx.x * (kIdxHistBins / 256) + j];
            cs += __shfl_xor(cs, 1, 64);
            cs += __shfl_xor(cs, 2, 64);
            if ((threadIdx.x & 3) == 0 && cs) atomicAdd(&a.coarse[r * 64 + threadIdx.x / 4], cs);
        }
    }
}

// --------------------------------------------------------------- streaming top-k
// A row's candidate list holds (position << 32 | key) words in position order,
// key = float_key(score); keys below the row's bound lo never join it.  Until the
// list first fills, lo = 0 and every causal key joins.  A full list is cut: every
// key whose top 16 bits reach those of the K-th key is kept and lo becomes that
// 16-bit floor (a dropped or later key below it ranks behind K kept keys larger
// than it); if that leaves no room, the list is cut to the row's exact top K
// (score descending, position ascending) and lo becomes the K-th key + 1 (a later
// key equal to it ranks behind K listed keys at least as large with smaller
// positions).  The end of the row takes the exact cut.
// One wave owns a row.  The list lives in global memory (it stays in L2); before
// reading it back the wave waits for its own stores and invalidates its vector
// L1 (an agent-scope acquire-release fence), so plain loads see the list.

// Number of set bits of a wave mask in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}


// Cuts list c[0, n), n >= K, in place (order kept).  Radix select over 8-bit
// digits with a 256-bin histogram in the wave's own LDS words, then one ordered
// compaction (ballot prefixes).  With EXACT the list keeps exactly the top K and
// the K-th largest key tau is returned; otherwise only the top 16 bits of tau are
// resolved and every key at or above lo = (those bits << 16) is kept (at least K
// keys), lo being returned: each dropped key is then below K kept ones.  *kept
// receives the new length.
template <int kCutBatch, bool EXACT>  // list entries per lane in flight
__device__ __forceinline__ uint32_t cut_to_topk(uint64_t* c, int n, int K, uint32_t* hist, int lane, int* kept)
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(c);  // low word of each entry
    uint32_t prefix = 0, pmask = 0;
    int want = K;  // rank of the K-th key among keys that match the prefix
    for (int shift = 24; shift >= (EXACT ? 0 : 16); shift -= 8) {
        for (int i = lane; i < 256; i += 64) hist[i] = 0u;
        for (int base = 0; base < n; base += 64 * kCutBatch) {
            uint32_t k[kCutBatch];
#pragma unroll
            for (int u = 0; u < kCutBatch; ++u) {
                const int i = min(base + 64 * u + lane, n - 1);
                k[u] = keys[2 * i];
            }
#pragma unroll
            for (int u = 0; u < kCutBatch; ++u)
                if (base + 64 * u + lane < n && (k[u] & pmask) == prefix) atomicAdd(&hist[(k[u] >> shift) & 255u], 1u);
        }
        uint32_t hb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hb[j] = hist[4 * lane + j];
        const uint32_t s = hb[0] + hb[1] + hb[2] + hb[3];
        uint32_t suf = s;  // keys in the bins of this and higher lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_down(suf, o, 64);
            if (lane + o < 64) suf += t;
        }
        uint32_t cum = suf - s;  // keys in higher digits than this lane's bins
        int d = -1;
        uint32_t above = 0;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (d < 0 && cum < (uint32_t)want && cum + hb[j] >= (uint32_t)want) {
                d = 4 * lane + j;
                above = cum;
            }
            cum += hb[j];
        }
        const uint64_t m = __ballot(d >= 0);
        const int src = __ffsll((unsigned long long)m) - 1;
        d = __shfl(d, src, 64);
        above = __shfl(above, src, 64);
        prefix |= (uint32_t)d << shift;
        pmask |= 0xFFu << shift;
        want -= (int)above;
    }
    // EXACT: keep every key above the K-th and the first `want` keys equal to it;
    // else every key whose top 16 bits are at least the prefix.  A batch is read
    // whole before any of it is written, and writes never pass the entries read.
    int out = 0, eq_seen = 0;
    for (int base = 0; base < n; base += 64 * kCutBatch) {
        uint64_t e[kCutBatch];
#pragma unroll
        for (int u = 0; u < kCutBatch; ++u) e[u] = c[min(base + 64 * u + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < kCutBatch; ++u) {
            const bool in = base + 64 * u + lane < n;
            const uint32_t k = (uint32_t)e[u];
            const bool gt = in && (EXACT ? k > prefix : k >= prefix), eq = EXACT && in && k == prefix;
            const uint64_t be = __ballot(eq);
            const bool keep = gt || (eq && eq_seen + lanes_below(be) < want);
            const uint64_t bk = __ballot(keep);
            if (keep) c[out + lanes_below(bk)] = e[u];
            out += __popcll(bk);
            eq_seen += __popcll(be);
        }
    }
    *kept = out;
    return __builtin_amdgcn_readfirstlane(prefix);
}

// ------------------------------------------------- final select of a candidate list
// The end of a fused row: its list (n > K entries in position order) is cut to the
// row's exact top K by the whole block.  The keys are staged in LDS with one load
// per entry (all of a thread's loads in flight at once; word j at j + j/32, so the
// per-thread segments below read without bank conflicts), three radix passes (11,
// 11 and 10 bits) find the K-th largest key tau and how many keys equal to it to
// take (the first ones in list order: the smallest positions), and an ordered
// compaction over contiguous per-thread segments writes the positions.
constexpr int kSelStage = 8192;                       // longest list staged in LDS
constexpr int kSelPad = kSelStage + kSelStage / 32;   // with one pad word per 32

__device__ __forceinline__ int sel_slot(int j) { return j + (j >> 5); }

// Exclusive prefix sum over the 256 threads of a block (tmp: 4 words of LDS).
__device__ __forceinline__ uint32_t block_excl_scan256(uint32_t v, uint32_t* tmp)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += tmp[w];
    __syncthreads();
    return base + x - v;
}

// Top K (score descending, position ascending) of list[0, n), K < n <= kSelStage,
// by all 256 threads; positions to dst[0, K) in ascending order.
__device__ __forceinline__ void block_select_list(const uint64_t* list, int n, int K, int32_t* dst, uint32_t* keys,
                                                  uint32_t* hist, uint32_t* tmp)
{
    const int tid = threadIdx.x;
    constexpr int PER = kSelStage / 256;
    {
        uint64_t e[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) e[i] = list[min(tid + 256 * i, n - 1)];
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (tid + 256 * i < n) keys[sel_slot(tid + 256 * i)] = (uint32_t)e[i];
    }
    __syncthreads();
    uint32_t prefix = 0, pmask = 0;
    int want = K;  // rank of the K-th key among the keys that match the prefix
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < 2048; i += 256) hist[i] = 0u;
        __syncthreads();
        for (int j = tid; j < n; j += 256) {
            const uint32_t k = keys[sel_slot(j)];
            if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins [hi - per, hi), hi = nb - per * t: the highest bins first
        const int per = nb / 256;
        const int hi = nb - per * tid;
        uint32_t sum = 0;
        for (int i = 0; i < per; ++i) sum += hist[hi - 1 - i];
        const uint32_t above = block_excl_scan256(sum, tmp);
        if (above < (uint32_t)want && above + sum >= (uint32_t)want) {
            uint32_t acc = above;
            int d = hi - 1;
            for (int i = 0; i < per; ++i) {
                const uint32_t h = hist[hi - 1 - i];
                if (acc + h >= (uint32_t)want) {
                    d = hi - 1 - i;
                    break;
                }
                acc += h;
            }
            tmp[4] = (uint32_t)d;
            tmp[5] = acc;
        }
        __syncthreads();
        want -= (int)tmp[5];
        prefix |= tmp[4] << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }
    const uint32_t tau = prefix;
    // ordered compaction: thread t takes entries [t*S, (t+1)*S)
    const int S = (n + 255) / 256;
    const int j0 = min(n, tid * S), j1 = min(n, j0 + S);
    int32_t pos[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) pos[i] = (int32_t)(list[min(j0 + i, n - 1)] >> 32);
    uint32_t gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t k = keys[sel_slot(j)];
        gt += k > tau;
        eq += k == tau;
    }
    const uint32_t before = block_excl_scan256((gt << 16) | eq, tmp);
    const int eq_before = (int)(before & 0xFFFFu);
    int out = (int)(before >> 16) + min(eq_before, want);
    int eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (j0 + i < j1) {
            const uint32_t k = keys[sel_slot(j0 + i)];
            bool take = k > tau;
            if (k == tau) take = eq_seen++ < want;
            if (take) dst[out++] = pos[i];
        }
    }
}

// ---------------------------------------------------- prefill tiling, 16x16 products
constexpr int kPrefillQPW = 2;
constexpr int kPrefillTK = 64;  // keys per LDS tile

template <int DT, int D, int HT, bool SEL>
__global__ __launch_bounds__(256, (SEL && DT != kF32) ? 2 : 1) void indexer_prefill_kernel(IndexerArgs a)
{
    constexpr int QPW = kPrefillQPW;
    constexpr int QPB = 4 * QPW;
    constexpr int TK = kPrefillTK;
    constexpr int NCH = Share<DT, D>::nch;
    constexpr int EB = ElemBytes<DT>::v;
    constexpr int ROWB = D * EB;          // bytes of a key row
    constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
    constexpr int PITCH = ROWB + 16;      // padded LDS row pitch (conflict-free 16-lane reads)
    constexpr int NLD = TK * CPR / 256;   // chunks each thread stages per tile
    static_assert(NLD >= 1 && (TK * CPR) % 256 == 0, "tile must split evenly over 256 threads");
    __shared__ __attribute__((aligned(16))) char smem[2][TK * PITCH];
    __shared__ uint32_t shist[SEL ? 4 : 1][256];
    __shared__ uint32_t sel_keys[SEL ? kSelPad : 1];
    __shared__ uint32_t sel_hist[SEL ? 2048 : 1];
    __shared__ uint32_t sel_tmp[8];
    __shared__ int sel_cnt[SEL ? QPB : 1];

    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.y;
    const int qb = gridDim.x - 1 - blockIdx.x;  // longest rows first
    clear_words(a);
    const int L = seq_len(a, b);
    const int t_end = a.t_begin + a.t_count;
    const int t0 = a.t_begin + qb * QPB;
    const int t_last = min(t0 + QPB, t_end) - 1;
    const int kend_blk = max(0, min(a.Lmax, L - a.T + t_last + 1));

    int tq[QPW], pq[QPW];
    bool vq[QPW];
    int kend_w = 0;
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
        tq[q] = t0 + wave * QPW + q;
        vq[q] = tq[q] < t_end;
        pq[q] = vq[q] ? L - a.T + tq[q] : -1;
        kend_w = max(kend_w, pq[q] + 1);
    }
    u32x4 qa[QPW][HT][NCH];
    float wv[QPW][HT][4];
#pragma unroll
    for (int q = 0; q < QPW; ++q) load_query<DT, D, HT>(a, b, vq[q] ? tq[q] : a.t_begin, vq[q], qa[q], wv[q]);
    // streaming top-k state of the wave's rows (wave-uniform)
    uint64_t* cand[QPW];
    int cnt[QPW];
    uint32_t lo[QPW];  // smallest key that still joins the list
    if constexpr (SEL) {
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            const int r = b * a.t_count + (vq[q] ? tq[q] - a.t_begin : 0);
            cand[q] = reinterpret_cast<uint64_t*>(a.sel_cand) + (size_t)r * a.sel_cap;
            cnt[q] = 0;
            lo[q] = 0u;
        }
    }

    const char* kbase = (const char*)a.k + (size_t)b * a.Lmax * ROWB;
    const int ntile = (kend_blk + TK - 1) / TK;
    // Bounded buffer accesses keep a tile free of branches: rows at or past
    // kend_blk load as zero, and a store is dropped when its offset lies past
    // the end of its row (keys after the query's position, lanes of groups 1-3).
    const buf_rsrc krs = make_rsrc(kbase, kend_blk * ROWB);
    buf_rsrc ksr = make_rsrc(a.k_scale + (DT == kFP8 ? (size_t)b * a.Lmax : 0), DT == kFP8 ? kend_blk * 4 : 0);
    buf_rsrc orow[QPW];
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
        if constexpr (SEL)
            orow[q] = make_rsrc(cand[q], vq[q] ? a.sel_cap * 8 : 0);
        else
            orow[q] = make_rsrc(a.scores + b * a.ld_b + (long long)((vq[q] ? tq[q] : a.t_begin) - a.t_begin) * a.ld_t,
                                vq[q] ? max(pq[q] + 1, 0) * 4 : 0);
    }
    u32x4 st[NLD];
    auto fetch = [&](int tile) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = threadIdx.x + 256 * i;
            st[i] = buf_ld16(krs, (tile * TK + c / CPR) * ROWB + (c % CPR) * 16);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int c = threadIdx.x + 256 * i;
            *reinterpret_cast<u32x4*>(&smem[buf][(c / CPR) * PITCH + (c % CPR) * 16]) = st[i];
        }
    };
    // Pieces of one 16-key sub-tile: its key operands, the contraction of one
    // row against them, and that row's epilogue (relu, weighted head sum, store
    // or list append).
    auto load_kb = [&](int buf, int kb0, u32x4 (&kb)[NCH], float& ks) {
        const char* rowp = &smem[buf][((kb0 & (TK - 1)) + n) * PITCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) kb[c] = *reinterpret_cast<const u32x4*>(rowp + Share<DT, D>::off(g, c));
        ks = 1.f;
        if constexpr (DT == kFP8) ks = __uint_as_float(buf_ld4(ksr, g == 0 ? (kb0 + n) * 4 : kDropOffset));
    };
    auto contract = [&](int q, const u32x4 (&kb)[NCH], f32x4 (&acc)[HT]) {
#pragma unroll
        for (int m = 0; m < HT; ++m) acc[m] = dot_share<DT, NCH>(qa[q][m], kb, f32x4{0, 0, 0, 0});
    };
    auto epilogue = [&](int q, int kb0, float ks, const f32x4 (&acc)[HT]) {
        const int key = kb0 + n;
        const float v = head_sum<HT>(acc, wv[q]);
        if constexpr (SEL) {
            const uint32_t kk = float_key(v * ks);
            const bool app = g == 0 && key <= pq[q] && kk >= lo[q];
            const uint64_t m = __ballot(app);
            buf_st8(orow[q], app ? (cnt[q] + lanes_below(m)) * 8 : kDropOffset, kk, (uint32_t)key);
            cnt[q] += __popcll(m);
        } else {
            buf_st4(orow[q], g == 0 ? key * 4 : kDropOffset, __float_as_uint(v * ks));
        }
    };
    // One MFMA, then up to three other vector instructions, over a stage: the
    // epilogue of one row fills the matrix core's shadow while the other row's
    // products run.
    // (Not for the fp32 operands, whose many small products make the ordering
    // costly to compile and which no long-context shape uses.)
    auto interleave = [&]() {
        if constexpr (DT != kF32) {
#pragma unroll
            for (int i = 0; i < HT * NCH * (DT == kFP8 ? 2 : 1); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
        }
    };
    // A whole tile, the two rows software-pipelined: the products of row 1 on
    // sub-tile j run beside the epilogue of row 0 on j, those of row 0 on j + 1
    // beside the epilogue of row 1 on j.
    auto score_tile = [&](int buf, int tile0) {
        static_assert(QPW == 2, "the pipeline alternates two rows");
        u32x4 kb[NCH], kn[NCH];
        float ks, ksn;
        f32x4 acc0[HT], acc1[HT];
        load_kb(buf, tile0, kb, ks);
        contract(0, kb, acc0);
#pragma unroll
        for (int sub = 0; sub < TK / 16; ++sub) {
            const int kb0 = tile0 + 16 * sub;
            contract(1, kb, acc1);
            epilogue(0, kb0, ks, acc0);
            interleave();
            if (sub + 1 < TK / 16) {
                load_kb(buf, kb0 + 16, kn, ksn);
                contract(0, kn, acc0);
            }
            epilogue(1, kb0, ks, acc1);
            if (sub + 1 < TK / 16) {
                interleave();
#pragma unroll
                for (int c = 0; c < NCH; ++c) kb[c] = kn[c];
                ks = ksn;
            }
        }
    };
    // A partial (diagonal) tile, sub-tile by sub-tile.
    auto score_sub = [&](int buf, int kb0) {
        u32x4 kb[NCH];
        float ks;
        load_kb(buf, kb0, kb, ks);
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            f32x4 acc[HT];
            contract(q, kb, acc);
            epilogue(q, kb0, ks, acc);
        }
    };

    if (ntile > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntile) fetch(it + 1);
        const int tile0 = it * TK;
        if constexpr (SEL) {
            // room for a whole tile of appends (TK per row) before it is scored;
            // one inlined cut serves both rows (operands picked, not indexed)
            static_assert(QPW == 2, "the cut below picks between two rows");
            // The cut first resolves 16 bits of the K-th key only; when the keys
            // sharing them leave no room, the exact cut follows.
            for (;;) {
                const bool c0 = tile0 <= pq[0] && cnt[0] + TK > a.sel_cap;
                const bool c1 = tile0 <= pq[1] && cnt[1] + TK > a.sel_cap;
                if (!c0 && !c1) break;
                uint64_t* c = c0 ? cand[0] : cand[1];
                int n = c0 ? cnt[0] : cnt[1];
                uint32_t l = cut_to_topk<4, false>(c, n, a.sel_k, shist[wave], lane, &n);
                if (n + TK > a.sel_cap) {
                    const uint32_t t = cut_to_topk<4, true>(c, n, a.sel_k, shist[wave], lane, &n);
                    l = t == 0xFFFFFFFFu ? t : t + 1u;  // strictly above the K-th key
                }
                if (c0) {
                    lo[0] = l;
                    cnt[0] = n;
                } else {
                    lo[1] = l;
                    cnt[1] = n;
                }
            }
        }
        if (tile0 + TK <= kend_w) {
            score_tile(buf, tile0);
        } else {
            for (int kb0 = tile0; kb0 < kend_w; kb0 += 16) score_sub(buf, kb0);
        }
        if (it + 1 < ntile) stash(buf ^ 1);
        __syncthreads();
    }

    if constexpr (SEL) {
        // The rows' lists are cut to their top K by the whole block, one row at a
        // time (lists past the LDS stage: by their own wave, the mid-row cut's way).
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < QPW; ++q) sel_cnt[wave * QPW + q] = vq[q] ? cnt[q] : -1;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int r = 0; r < QPB; ++r) {
            const int nr = sel_cnt[r];
            if (nr < 0) continue;
            const int tr = t0 + r;
            uint64_t* list = reinterpret_cast<uint64_t*>(a.sel_cand) + (size_t)(b * a.t_count + tr - a.t_begin) * a.sel_cap;
            int32_t* dst = a.sel_idx + ((size_t)b * a.T + tr) * a.sel_k;
            if (nr <= a.sel_k) {
                for (int j = threadIdx.x; j < a.sel_k; j += 256) dst[j] = j < nr ? (int32_t)(list[j] >> 32) : -1;
            } else if (nr <= kSelStage) {
                block_select_list(list, nr, a.sel_k, dst, sel_keys, sel_hist, sel_tmp);
            } else if (r / QPW == wave) {
                int m = 0;
                cut_to_topk<16, true>(list, nr, a.sel_k, shist[wave], lane, &m);
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
                for (int j = lane; j < a.sel_k; j += 64) dst[j] = (int32_t)(list[j] >> 32);
            }
            __syncthreads();
        }
    } else if (a.fill) {
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            if (!vq[q]) continue;
            float* row = a.scores + b * a.ld_b + (long long)(tq[q] - a.t_begin) * a.ld_t;
            for (int s = max(pq[q] + 1, 0) + lane; s < a.Lmax; s += 64) row[s] = -INFINITY;
        }
    }
}

template <int DT, int D, int HT>
hipError_t launch_dt(const IndexerArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    if (a.t_count <= 2) {
        constexpr int NCH = Share<DT, D>::nch;
        // about 2048 persistent waves over the grid for bf16 keys, 3072 for fp8
        // (measured with non-temporal key loads: bf16 1536-4096, fp8 2048-4096
        // waves; fp8 64-key strips carry twice the products per byte); 8 KB strips
        // keep the window of rows in flight small (measured best among 4, 8 and 16 KB)
        const int waves = DT == kFP8 ? 3072 : 2048;
        const int per_seq = (int)((waves + 4LL * a.B - 1) / (4LL * a.B));
        if (a.t_count == 1) {
            constexpr int TPW = NCH >= 8 ? 1 : 8 / NCH;
            const int strips = (a.Lmax + TPW * 16 - 1) / (TPW * 16);
            dim3 grid(std::max(1, std::min(per_seq, (strips + 3) / 4)), 1, a.B);
            indexer_decode_kernel<DT, D, HT, 1, TPW><<<grid, 256, 0, s>>>(a);
        } else {
            constexpr int TPW = NCH >= 8 ? 1 : 8 / NCH;
            const int strips = (a.Lmax + TPW * 16 - 1) / (TPW * 16);
            dim3 grid(std::max(1, std::min(per_seq, (strips + 3) / 4)), 1, a.B);
            indexer_decode_kernel<DT, D, HT, 2, TPW><<<grid, 256, 0, s>>>(a);
        }
    } else {
        constexpr int QPB = 4 * kPrefillQPW;
        dim3 grid((a.t_count + QPB - 1) / QPB, a.B);
        indexer_prefill_kernel<DT, D, HT, false><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int DT, int D, int HT>
hipError_t launch_sel_dt(const IndexerArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    constexpr int QPB = 4 * kPrefillQPW;
    dim3 grid((a.t_count + QPB - 1) / QPB, a.B);
    indexer_prefill_kernel<DT, D, HT, true><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_sel_heads(const IndexerArgs& a, hipStream_t s)
{
    return a.H <= 16 ? launch_sel_dt<DT, D, 1>(a, s) : launch_sel_dt<DT, D, 4>(a, s);
}

template <int DT, int D>
hipError_t launch_heads(const IndexerArgs& a, hipStream_t s)
{
    return a.H <= 16 ? launch_dt<DT, D, 1>(a, s) : launch_dt<DT, D, 4>(a, s);
}

}  // namespace

bool indexer_supported(int dtype, int D, int H)
{
    if (H < 1 || H > 64) return false;
    if (dtype == kF32) return D == 32 || D == 64 || D == 128;
    if (dtype == kBF16 || dtype == kFP8) return D == 128;
    return false;
}

int index_topk_cap(int K)
{
    const int c = std::max(4 * K, K + 64);
    return (c + 63) / 64 * 64;
}

hipError_t launch_index_topk(int dtype, const IndexerArgs& a, hipStream_t s)
{
    if (a.sel_k < 1 || a.sel_cap < a.sel_k + kPrefillTK) return hipErrorInvalidValue;
    if (dtype == kBF16) return launch_sel_heads<kBF16, 128>(a, s);
    if (dtype == kFP8) return launch_sel_heads<kFP8, 128>(a, s);
    if (a.D == 32) return launch_sel_heads<kF32, 32>(a, s);
    if (a.D == 64) return launch_sel_heads<kF32, 64>(a, s);
    return launch_sel_heads<kF32, 128>(a, s);
}

hipError_t launch_indexer(int dtype, const IndexerArgs& a, hipStream_t s)
{
    if (dtype == kBF16) return launch_heads<kBF16, 128>(a, s);
    if (dtype == kFP8) return launch_heads<kFP8, 128>(a, s);
    if (a.D == 32) return launch_heads<kF32, 32>(a, s);
    if (a.D == 64) return launch_heads<kF32, 64>(a, s);
    return launch_heads<kF32, 128>(a, s);
}

}  // namespace dsa
