// sparse_mla_bwd.hip -- backward of the sparse absorbed-latent MLA on gfx950.
//
// DeepSeek-V3.2 model documentation, model description: DSA is trainable.  For
// the forward of sparse_mla.hip (z_j = sm q . k_j over a query's selected rows,
// o = softmax(z) . v, lse its log-sum-exp) and an incoming gradient dO, the
// gradients are
//   dP_j = dO . v_j,   p_j = e^(z_j - lse),   D = dO . o = sum_j p_j dP_j,
//   dz_j = p_j (dP_j - D),
//   dq = sm sum_j dz_j k_j,   dkv[idx_j] += sm dz_j q  (all columns)  + p_j dO  (value columns).
// D is summed from the recomputed p and dP rather than taken from the bf16
// output: with a concentrated softmax dz is a small difference, and the output's
// rounding (relative 2^-9 per element) would otherwise dominate dq.
// Four launches per query chunk:
//   prep    q and dO transposed to head-minor rows (heads padded to 16 with
//           zeros) for the dkv contraction; dq cleared when the list is split;
//   scores  one 512-thread workgroup per (query, split, 128 heads): the forward's
//           gather and contraction-split logits, a second contraction
//           dP^T = V . dO^T, p from the forward's lse; p and dP stored per
//           (list entry, head) in fp32, the split's sum of p dP per head;
//   dq      D from the split sums, dz formed per entry, then the forward's value
//           sum run over all key columns with dz in place of p:
//           dq += dz . K (head rows, so a lane group writes 32 consecutive
//           columns of one head), split lists add with fp32 atomics;
//   dkv     per (query, split): for each 32-column block the key part
//           (sm dz^T q) and, below Dv, the value part (p^T dO) contract over the
//           heads into one accumulator on 32x32x16 MFMA per 32-entry tile, and
//           the block is added to the cache rows with fp32 atomics, or stored when
//           the call cleared dkv and no two (query, entry) pairs share a row (one
//           query per sequence, strictly increasing list).
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTK = 32;             // list entries per tile
constexpr int kMaxList = 4096;      // longest list a split holds in LDS
constexpr float kLog2eB = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ void bar_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void bar_lds_vm() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int DQK, int DV>
struct BwdCfg {
    static constexpr int ROWB = DQK * 2;
    static constexpr int CPR = DQK / 8;
    static constexpr int PCH = CPR + 1;
    static constexpr int PITCH = PCH * 16;
    static constexpr int TILE_CH = kTK * PCH;
    static constexpr int DMA_PER_WAVE = (TILE_CH + 511) / 512;
    static constexpr int BUF_CH = DMA_PER_WAVE * 512;
    static constexpr int HALF = DQK / 2, SHARE = DQK / 4, QS = SHARE / 8;   // q.k contraction split
    static constexpr int VHALF = DV / 2, VSHARE = DV / 4, VS = VSHARE / 8;  // dO.v contraction split
    static constexpr int QT = HALF / 32;                                     // dq tiles of a wave half
    static constexpr int NBK = DQK / 32, NBV = DV / 32;                      // dkv column blocks
    static_assert(DQK % 64 == 0 && DV % 64 == 0 && DV <= DQK && SHARE % 8 == 0 && VSHARE % 8 == 0, "shape");
};

using BwdArgs = MlaBwdArgs;

__device__ __forceinline__ int xcd_map(int L, int n)
{
    const int per = (n + 7) >> 3;
    return (L & 7) * per + (L >> 3);
}

// ---------------------------------------------------------------- clears
__global__ __launch_bounds__(256) void zero_kernel(float* p, long long n)
{
    const long long n4 = n / 4;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256)
        st16(p + 4 * i, u32x4{0u, 0u, 0u, 0u});
    for (long long i = 4 * n4 + (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        p[i] = 0.f;
}

// ---------------------------------------------------------------- prep
// Block (r, c) of 256 threads: chunk row r, 64-column slice c of [q | dO] (q
// columns first).  The slice of all Hp heads is staged in LDS and written back
// head-minor.  Blocks with c == 0 clear the row's dq when the list is split.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    __shared__ uint16_t tile[128][64 + 2];
    const int r = blockIdx.x, c = blockIdx.y;
    const int b = r / a.t_count, t = a.t_begin + r % a.t_count;
    const size_t grow = (size_t)b * a.T + t;
    const int tid = threadIdx.x;
    const bool isq = c * 64 < DQK;
    const int col0 = isq ? c * 64 : c * 64 - DQK;
    const int D = isq ? DQK : DV;
    const uint16_t* src = isq ? a.q : a.dout;
    // stage rows h (64 columns = 128 bytes: 8 lanes of 16 bytes per head)
    for (int i = tid; i < a.Hp * 8; i += 256) {
        const int h = i >> 3, k = i & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < a.H && col0 + 8 * k < D) v = ld16(src + (grow * a.H + h) * D + col0 + 8 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[h][8 * k + 2 * e] = (uint16_t)(v[e] & 0xFFFFu);
            tile[h][8 * k + 2 * e + 1] = (uint16_t)(v[e] >> 16);
        }
    }
    __syncthreads();
    uint16_t* dst = isq ? a.qT + (size_t)r * DQK * a.Hp : a.dT + (size_t)r * DV * a.Hp;
    for (int i = tid; i < 64 * a.Hp; i += 256) {
        const int d = i / a.Hp, h = i - d * a.Hp;
        if (col0 + d < D) dst[(size_t)(col0 + d) * a.Hp + h] = tile[h][d];
    }
    if (c == 0 && a.n_split > 1) {
        // split lists add their dq with atomics: clear the row first
        float* dqr = a.dq + grow * a.H * DQK;
        for (int i = tid; i < a.H * DQK / 4; i += 256) st16(dqr + 4 * i, u32x4{0u, 0u, 0u, 0u});
    }
}

// ---------------------------------------------------------------- list set-up
// Loads the split's index list into LDS as row byte offsets (lrow, row 0 for
// skipped entries) and/or cache rows (lsrc, -1 for skipped entries), and the
// validity mask of each 32-entry tile.
template <class C>
__device__ __forceinline__ void load_list(const int32_t* idxr, int j_begin, int j_end, int n_list, int L,
                                          uint32_t* lrow, int32_t* lsrc, uint32_t* tmask, int tid, int lane)
{
    constexpr int PER = kMaxList / 512;
    const int j_last = max(j_end - 1, 0);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int j = tid + 512 * r;
        const int s = idxr[min(j_begin + j, j_last)];
        const bool ok = j < n_list && j_begin + j < j_end && s >= 0 && s < L;
        if (lrow) lrow[j] = ok ? (uint32_t)s * C::ROWB : 0u;
        if (lsrc) lsrc[j] = ok ? s : -1;
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {
            tmask[j / kTK] = (uint32_t)bits;
            tmask[j / kTK + 1] = (uint32_t)(bits >> 32);
        }
    }
}

// Direct loads of list tile [j0, j0 + 32) into dst (whole rows, padded pitch;
// the pad chunk and the tail fetch rows of the tile so every wave issues the
// same number of loads). A class member rather than a free function template:
// hipcc's host pass rejects a second kernel's call of the free template.
template <class C>
struct RowGather {
    static __device__ __forceinline__ void run(const char* kvb, const uint32_t* lrow, int j0, int w, int lane, u32x4* dst)
    {
        constexpr int DR = 512 / C::PCH, DCH = 512 % C::PCH;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int wu = __builtin_amdgcn_readfirstlane(w);
        int r = (wu * 64 + ln) / C::PCH;
        int c = wu * 64 + ln - r * C::PCH;
        uint32_t roff[C::DMA_PER_WAVE], coff[C::DMA_PER_WAVE];
    #pragma unroll
        for (int k = 0; k < C::DMA_PER_WAVE; ++k) {
            roff[k] = lrow[j0 + min(r, kTK - 1)];
            coff[k] = c == C::CPR ? 0u : (uint32_t)c * 16u;
            r += DR;
            c += DCH;
            if (c >= C::PCH) {
                c -= C::PCH;
                ++r;
            }
        }
    #pragma unroll
        for (int k = 0; k < C::DMA_PER_WAVE; ++k)
            __builtin_amdgcn_global_load_lds(kvb + (roff[k] + coff[k]),
                                             (__attribute__((address_space(3))) void*)(dst + (wu + 8 * k) * 64), 16, 0, 0);
    }
};

struct Unit {
    int hb, split, rq, b, t, L, j_begin, j_end, n_tiles;
    size_t grow;  // b * T + t
    bool valid;
};

__device__ __forceinline__ Unit unit_of(const BwdArgs& a, int per_hb)
{
    Unit u;
    const int HB = per_hb;
    const int n_units = a.B * a.t_count * a.n_split * HB;
    const int unit = xcd_map(blockIdx.x, n_units);
    u.valid = unit < n_units;
    const int un = u.valid ? unit : 0;
    u.hb = un % HB;
    u.split = (un / HB) % a.n_split;
    u.rq = un / HB / a.n_split;
    u.b = u.rq / a.t_count;
    u.t = a.t_begin + u.rq % a.t_count;
    u.grow = (size_t)u.b * a.T + u.t;
    u.L = min(a.kv_len[u.b], a.Lmax);
    const int per = ((a.K + a.n_split - 1) / a.n_split + kTK - 1) / kTK * kTK;
    u.j_begin = u.split * per;
    u.j_end = min(a.K, u.j_begin + per);
    u.n_tiles = (u.j_end > u.j_begin && u.L > 0) ? (u.j_end - u.j_begin + kTK - 1) / kTK : 0;
    return u;
}

// ---------------------------------------------------------------- scores
// Wave (pair p, half h): heads 32p .. 32p + 31 of the block, contraction half h
// of q.k and of dO.v.  Lane holds keys 8*i + 4*kb + j (register 4*i + j) of
// head `col` after the two halves are summed through LDS.
template <int DQK, int DV>
__global__ __launch_bounds__(512) void bwd_scores_kernel(BwdArgs a)
{
    using C = BwdCfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) u32x4 tA[C::BUF_CH];
    __shared__ __attribute__((aligned(16))) u32x4 tB[C::BUF_CH];
    __shared__ float xbuf[8][16][64];
    __shared__ uint32_t lrow[kMaxList];
    __shared__ uint32_t tmask[kMaxList / kTK];

    const Unit u = unit_of(a, (a.H + 127) / 128);
    if (!u.valid) return;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int pair = w >> 1, half = w & 1;
    const int col = lane & 31, kb = lane >> 5;
    const int head = u.hb * 128 + pair * 32 + col;
    const bool head_ok = head < a.H;
    const size_t qrow = u.grow * a.H + (head_ok ? head : 0);
    const int r = u.b * a.t_count + (u.t - a.t_begin);  // chunk row

    load_list<C>(a.idx + u.grow * a.K, u.j_begin, u.j_end, u.n_tiles * kTK, u.L, lrow, nullptr, tmask, tid, lane);
    u32x4 qb[C::QS], ob[C::VS];
    {
        const uint16_t* qs = a.q + qrow * DQK + C::HALF * half + C::SHARE * kb;
        const uint16_t* os = a.dout + qrow * DV + C::VHALF * half + C::VSHARE * kb;
#pragma unroll
        for (int s = 0; s < C::QS; ++s) qb[s] = ld16(qs + 8 * s);
#pragma unroll
        for (int s = 0; s < C::VS; ++s) ob[s] = ld16(os + 8 * s);
    }
    const float zc = a.sm * kLog2eB;
    const float lse_h = a.lse[qrow];
    const float l2 = lse_h * kLog2eB;
    const bool live = head_ok && lse_h != -INFINITY;
    float dsum = 0.f;  // this lane's share of sum_j p_j dP_j
    bar_lds();

    const char* kvb = (const char*)a.kv + (size_t)u.b * a.Lmax * C::ROWB;
    float* store = (half == 0 ? a.P : a.DP) + (size_t)r * a.K * a.Hp;
    const bool store_head = head < a.Hp;  // padded heads get zeros
    if (u.n_tiles > 0) RowGather<C>::run(kvb, lrow, 0, w, lane, tA);
#pragma unroll 1
    for (int it = 0; it < u.n_tiles; ++it) {
        bar_lds_vm();
        const u32x4* tile = (it & 1) ? tB : tA;
        if (it + 1 < u.n_tiles) RowGather<C>::run(kvb, lrow, (it + 1) * kTK, w, lane, (it & 1) ? tA : tB);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t vm = tmask[it];
        const char* tb = reinterpret_cast<const char*>(tile);
        f32x16 sacc, dacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = dacc[e] = 0.f;
        const char* kr = tb + col * C::PITCH + (C::HALF * half + C::SHARE * kb) * 2;
#pragma unroll
        for (int s = 0; s < C::QS; ++s) sacc = mfma32(*reinterpret_cast<const u32x4*>(kr + 16 * s), qb[s], sacc);
        const char* vr = tb + col * C::PITCH + (C::VHALF * half + C::VSHARE * kb) * 2;
#pragma unroll
        for (int s = 0; s < C::VS; ++s) dacc = mfma32(*reinterpret_cast<const u32x4*>(vr + 16 * s), ob[s], dacc);
#pragma unroll
        for (int e = 0; e < 16; ++e) xbuf[w][e][lane] = sacc[e];
        bar_lds();
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] += xbuf[w ^ 1][e][lane];
        bar_lds();
#pragma unroll
        for (int e = 0; e < 16; ++e) xbuf[w][e][lane] = dacc[e];
        bar_lds();
        const int j0 = u.j_begin + it * kTK;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            const float dp = dacc[e] + xbuf[w ^ 1][e][lane];
            const bool ok = live && ((vm >> key) & 1u);
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sacc[e], zc, -l2)) : 0.f;
            const float d = ok ? dp : 0.f;
            dsum = fmaf(p, d, dsum);
            if (store_head && j0 + key < u.j_end) store[(size_t)(j0 + key) * a.Hp + head] = half == 0 ? p : d;
        }
    }
    dsum += __shfl_xor(dsum, 32);
    if (half == 0 && kb == 0 && store_head) a.Dd[((size_t)r * a.n_split + u.split) * a.Hp + head] = dsum;
}

// ---------------------------------------------------------------- dq
// Wave (pair p, half h): heads 32p.., key columns [HALF * h, + HALF) of dq.
// dz is the A operand, formed per lane in the logit register layout (lane: head
// `col`, entries 8*i + 4*kb + jj) from the stored p and dP and D, the sum of the
// split sums; K comes through transposed LDS reads as the B operand.
template <int DQK, int DV>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a)
{
    using C = BwdCfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) u32x4 tA[C::BUF_CH];
    __shared__ __attribute__((aligned(16))) u32x4 tB[C::BUF_CH];
    __shared__ uint32_t lrow[kMaxList];
    __shared__ uint32_t tmask[kMaxList / kTK];

    const Unit u = unit_of(a, (a.H + 127) / 128);
    if (!u.valid) return;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int pair = w >> 1, half = w & 1;
    const int col = lane & 31, kb = lane >> 5;
    const int head = u.hb * 128 + pair * 32 + col;
    const int r = u.b * a.t_count + (u.t - a.t_begin);

    load_list<C>(a.idx + u.grow * a.K, u.j_begin, u.j_end, u.n_tiles * kTK, u.L, lrow, nullptr, tmask, tid, lane);
    bar_lds();
    f32x16 acc[C::QT];
#pragma unroll
    for (int v = 0; v < C::QT; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[v][e] = 0.f;

    const char* kvb = (const char*)a.kv + (size_t)u.b * a.Lmax * C::ROWB;
    const int hc = head < a.Hp ? head : 0;
    const float* pr = a.P + (size_t)r * a.K * a.Hp + hc;
    const float* dpr = a.DP + (size_t)r * a.K * a.Hp + hc;
    float Dh = 0.f;
    for (int s = 0; s < a.n_split; ++s) Dh += a.Dd[((size_t)r * a.n_split + s) * a.Hp + hc];
    const int grp = lane >> 4, m16 = lane & 15;
    const int kbv = grp >> 1, vb = 16 * (grp & 1);
    const int jr = m16 >> 2, qc = m16 & 3;
    if (u.n_tiles > 0) RowGather<C>::run(kvb, lrow, 0, w, lane, tA);
#pragma unroll 1
    for (int it = 0; it < u.n_tiles; ++it) {
        const int j0 = u.j_begin + it * kTK;
        // dz of keys 8*i + 4*kb + jj of head `col` (skipped entries are zero)
        float z[16], zp[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            const size_t o = (size_t)min(j0 + key, a.K - 1) * a.Hp;
            zp[e] = pr[o];
            z[e] = dpr[o];
        }
        bar_lds_vm();
        const uint32_t vm = tmask[it];
        const u32x4* tile = (it & 1) ? tB : tA;
        if (it + 1 < u.n_tiles) RowGather<C>::run(kvb, lrow, (it + 1) * kTK, w, lane, (it & 1) ? tA : tB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            z[e] = ((vm >> key) & 1u) ? zp[e] * (z[e] - Dh) : 0.f;
        }
        const char* tb = reinterpret_cast<const char*>(tile);
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            u32x4 pb;
            pb[0] = pack_bf16x2(z[8 * step + 0], z[8 * step + 1]);
            pb[1] = pack_bf16x2(z[8 * step + 2], z[8 * step + 3]);
            pb[2] = pack_bf16x2(z[8 * step + 4], z[8 * step + 5]);
            pb[3] = pack_bf16x2(z[8 * step + 6], z[8 * step + 7]);
            const char* r0 = tb + (16 * step + 4 * kbv + jr) * C::PITCH + (C::HALF * half + vb + 4 * qc) * 2;
            const char* r1 = r0 + 8 * C::PITCH;
#pragma unroll
            for (int v = 0; v < C::QT; ++v) {
                const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(r0 + 64 * v));
                const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(r1 + 64 * v));
                const u32x2 y0 = __builtin_bit_cast(u32x2, x0);
                const u32x2 y1 = __builtin_bit_cast(u32x2, x1);
                acc[v] = mfma32(pb, u32x4{y0[0], y0[1], y1[0], y1[1]}, acc[v]);
            }
        }
    }
    // lane holds column HALF*half + 32*v + col of heads 32*pair + 8*i + 4*kb + jj (register 4*i + jj)
    const int h0 = u.hb * 128 + pair * 32 + 4 * kb;
    float* dst = a.dq + (u.grow * a.H + h0) * DQK + C::HALF * half + col;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (h0 + 8 * i + jj >= a.H) continue;
            float* p = dst + (size_t)(8 * i + jj) * DQK;
#pragma unroll
            for (int v = 0; v < C::QT; ++v) {
                const float x = a.sm * acc[v][4 * i + jj];
                if (a.n_split == 1)
                    p[32 * v] = x;
                else
                    unsafeAtomicAdd(p + 32 * v, x);
            }
        }
}

// ---------------------------------------------------------------- dkv
// Per (query, split).  A value column c < DV of a cache row gets sm dz q (key part)
// and p dO (value part); both contractions over the heads share one accumulator,
// so each (entry, column) takes one atomic.  Main pass: wave w owns the 32-column
// blocks w and w + 8 below DV with their q and dO operands (head-minor rows from
// prep) in registers; per tile it forms its A operands, bf16 p and sm dz =
// sm p (dP - D), for entry row `col` of the tile, runs both contractions on
// 32x32x16 MFMA and adds each lane's 16 results (entries 8*i + 4*kb + jj, column
// `col`) to the cache rows with fp32 atomics.  Second pass: the key-only blocks
// (the rope columns at and past DV), tiles dealt round-robin over the waves.
template <int DQK, int DV>
__global__ __launch_bounds__(512) void bwd_dkv_kernel(BwdArgs a)
{
    using C = BwdCfg<DQK, DV>;
    constexpr int HS = 8;  // 16-head steps: up to 128 heads
    constexpr int NB = C::NBK, NV = C::NBV;
    constexpr int NR = NB - NV;  // key-only blocks
    static_assert(NV <= 16 && NR >= 1 && NR <= 2, "block split of the dkv kernel");
    __shared__ int32_t lsrc[kMaxList];
    __shared__ uint32_t lrow[kMaxList];
    __shared__ uint32_t tmask[kMaxList / kTK];
    __shared__ __attribute__((aligned(16))) float Ds[128];

    const Unit u = unit_of(a, 1);
    if (!u.valid) return;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int col = lane & 31, kb = lane >> 5;
    const int r = u.b * a.t_count + (u.t - a.t_begin);
    load_list<C>(a.idx + u.grow * a.K, u.j_begin, u.j_end, u.n_tiles * kTK, u.L, lrow, lsrc, tmask, tid, lane);
    if (tid < a.Hp) {
        float d = 0.f;
        for (int s = 0; s < a.n_split; ++s) d += a.Dd[((size_t)r * a.n_split + s) * a.Hp + tid];
        Ds[tid] = d;
    }
    // Exclusive rows: with one query per sequence, and the query's whole list made
    // of strictly increasing valid entries followed only by skipped ones (top-k's
    // layout), every cache row gets one update from one lane in the whole call.  When
    // dkv was cleared by this call, the blocks are then stored instead of added with
    // atomics (with accumulation the atomics stay: a load before each store would
    // make the wave wait on memory, which the no-return atomics do not).  Every
    // workgroup of the query reads the same list and so takes the same path.
    bool viol = a.T != 1 || a.accumulate;
    if (!viol) {
        const int32_t* full = a.idx + u.grow * a.K;
        for (int i = tid; i < a.K; i += 512) {
            const int s1 = full[i];
            const bool v1 = s1 >= 0 && s1 < u.L;
            if (i > 0 && v1) {
                const int s0 = full[i - 1];
                const bool v0 = s0 >= 0 && s0 < u.L;
                if (!v0 || s0 >= s1) viol = true;
            }
        }
    }
    const bool excl = !__syncthreads_or(viol);

    const uint16_t* qT = a.qT + (size_t)r * DQK * a.Hp;
    const uint16_t* dT = a.dT + (size_t)r * DV * a.Hp;
    const float* srcp = a.P + (size_t)r * a.K * a.Hp;
    const float* srcd = a.DP + (size_t)r * a.K * a.Hp;
    const int hs = a.Hp / 16;
    float* dkvb = a.dkv + (size_t)u.b * a.Lmax * DQK;

    // A operands of tile `it`: entry row `col`, heads 16 s + 8 kb .. + 8
    auto load_a = [&](int it, u32x4 (&ap)[HS], u32x4 (&az)[HS], bool want_p) {
        const size_t ao = (size_t)min(u.j_begin + it * kTK + col, a.K - 1) * a.Hp + 8 * kb;
#pragma unroll
        for (int s = 0; s < HS; ++s) {
            if (s < hs) {
                const u32x4 lo = ld16(srcp + ao + 16 * s), hi = ld16(srcp + ao + 16 * s + 4);
                const u32x4 dlo = ld16(srcd + ao + 16 * s), dhi = ld16(srcd + ao + 16 * s + 4);
                const f32x4 D0 = *reinterpret_cast<const f32x4*>(&Ds[16 * s + 8 * kb]);
                const f32x4 D1 = *reinterpret_cast<const f32x4*>(&Ds[16 * s + 8 * kb + 4]);
                float pv[8], z[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    pv[k] = __uint_as_float(lo[k]);
                    pv[4 + k] = __uint_as_float(hi[k]);
                    z[k] = a.sm * pv[k] * (__uint_as_float(dlo[k]) - D0[k]);
                    z[4 + k] = a.sm * pv[4 + k] * (__uint_as_float(dhi[k]) - D1[k]);
                }
                if (want_p)
                    ap[s] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                                  pack_bf16x2(pv[6], pv[7])};
                az[s] = u32x4{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]), pack_bf16x2(z[4], z[5]),
                              pack_bf16x2(z[6], z[7])};
            } else {
                ap[s] = u32x4{0u, 0u, 0u, 0u};
                az[s] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // B operand of column block blk: lane (column col, k-block kb) holds heads 16 s + 8 kb .. + 8
    auto load_b = [&](const uint16_t* opT, int blk, u32x4 (&bo)[HS]) {
#pragma unroll
        for (int s = 0; s < HS; ++s)
            bo[s] = s < hs ? ld16(opT + (size_t)(32 * blk + col) * a.Hp + 16 * s + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
    };
    auto add_rows = [&](int it, int blk, const f32x16& acc) {
        const uint32_t vm = tmask[it];
        if (excl) {  // every word of these rows is this lane's alone, and dkv was cleared: store
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
                const int row = lsrc[it * kTK + key];
                if (((vm >> key) & 1u) && row >= 0) dkvb[(size_t)row * DQK + 32 * blk + col] = acc[e];
            }
            return;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            const int row = lsrc[it * kTK + key];
            if (((vm >> key) & 1u) && row >= 0) unsafeAtomicAdd(dkvb + (size_t)row * DQK + 32 * blk + col, acc[e]);
        }
    };

    {  // main pass: blocks w and w + 8 below DV, key and value parts together
        u32x4 bq[2][HS], bv[2][HS];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int blk = min(w + 8 * i, NV - 1);
            load_b(qT, blk, bq[i]);
            load_b(dT, blk, bv[i]);
        }
#pragma unroll 1
        for (int it = 0; it < u.n_tiles && w < NV; ++it) {
            u32x4 ap[HS], az[HS];
            load_a(it, ap, az, true);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int blk = w + 8 * i;
                if (blk >= NV) break;
                f32x16 acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
                for (int s = 0; s < HS; ++s)
                    if (s < hs) {
                        acc = mfma32(az[s], bq[i][s], acc);
                        acc = mfma32(ap[s], bv[i][s], acc);
                    }
                add_rows(it, blk, acc);
            }
        }
    }
    {  // second pass: key-only blocks, tiles dealt over the waves
        u32x4 br[NR][HS];
#pragma unroll
        for (int i = 0; i < NR; ++i) load_b(qT, NV + i, br[i]);
#pragma unroll 1
        for (int it = w; it < u.n_tiles; it += 8) {
            u32x4 ap[HS], az[HS];
            load_a(it, ap, az, false);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                f32x16 acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
                for (int s = 0; s < HS; ++s)
                    if (s < hs) acc = mfma32(az[s], br[i][s], acc);
                add_rows(it, NV + i, acc);
            }
        }
    }
}

template <int DQK, int DV>
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s)
{
    const int rows = a.B * a.t_count;
    bwd_prep_kernel<DQK, DV><<<dim3(rows, (DQK + DV) / 64), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int HB = (a.H + 127) / 128;
    const long long units = (long long)rows * a.n_split * HB;
    const dim3 grid((unsigned)(8 * ((units + 7) / 8)));
    bwd_scores_kernel<DQK, DV><<<grid, 512, 0, s>>>(a);
    bwd_dq_kernel<DQK, DV><<<grid, 512, 0, s>>>(a);
    const long long units1 = (long long)rows * a.n_split;
    bwd_dkv_kernel<DQK, DV><<<dim3((unsigned)(8 * ((units1 + 7) / 8))), 512, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool mla_bwd_supported(int dtype, int Dqk, int Dv, int H)
{
    return dtype == kBF16 && H >= 1 && H <= 128 && ((Dqk == 576 && Dv == 512) || (Dqk == 192 && Dv == 128));
}

hipError_t launch_zero_f32(float* p, long long n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((n / 4 + 255) / 256 + 1, 4096);
    zero_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_mla_bwd_chunk(const MlaBwdArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    if (a.Dqk == 192) return launch_bwd_chunk<192, 128>(a, s);
    return launch_bwd_chunk<576, 512>(a, s);
}

}  // namespace dsa
