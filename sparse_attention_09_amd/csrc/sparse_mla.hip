// sparse_mla.hip -- sparse absorbed-latent MLA forward on gfx950 MFMA.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 2:
// main MLA attention runs only over each query's selected tokens, which with a
// sparse kernel costs O(index_topk) per query instead of O(L).  Absorbed form:
// one latent row kv[s] = [c_kv (Dv) | k_rope] is the key of every head and its
// first Dv columns are the value, so all heads of a query share each gathered
// row:  z_j = sm_scale * q_h . kv[idx_j],  o_h = sum_j softmax(z)_j kv[idx_j, :Dv].
//
// bf16 kernel (the DeepSeek shapes).  One 512-thread workgroup owns a
// (query, split of the index list) unit and all 128 heads, so every selected
// row is gathered once per query.  Per 32-entry tile:
//   - the rows are gathered straight into LDS (global_load_lds, 16 B per lane,
//     whole rows, double buffered: tile t+1 is in flight while t is computed);
//   - wave pair p (heads 32p..32p+31) splits the contraction: wave (p, h)
//     computes S^T_h[32 keys x 32 heads] = K[:, d-half h] . Q^T[d-half h] on
//     32x32x16 MFMA (keys on M, heads on N), the halves are summed through LDS,
//     and both waves run the same online softmax in registers;
//   - wave (p, h) then accumulates O^T[value half h (Dv/2) x 32 heads] +=
//     V^T . P^T, P^T taken straight from the logit registers (the key order of
//     the contraction is permuted to match) and V^T read from the row-major tile
//     with the LDS transpose load.
// Thirty-two heads per wave halve the LDS bytes per MFMA flop against 16, and
// the contraction split keeps two waves per SIMD.  Units of consecutive
// queries go to one XCD, whose L2 then serves rows that neighbouring queries
// share.  Each workgroup writes one row per head (the output row, or for a
// split its value row divided by its own softmax sum plus the running max and
// sum), staged through LDS so that rows leave as whole contiguous writes; a
// log-sum-exp combine kernel merges the splits.
//
// fp32 kernel (small shapes only): 16 heads per wave on 16x16x4 MFMA, the
// gathered tile staged through registers.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTileKeys = 32;
// A split's partial result for one (query, head): its value row, then the running max m
// (log2 domain) and sum l, padded to 16 bytes.  fp32 outputs keep the unnormalised
// fp32 value row; bf16 outputs keep the row already divided by l, in bf16 (the final
// output is bf16 too), which halves the partial traffic of split queries.
template <int DT, int DV> struct PartRow {
    static constexpr int vbytes = DV * (DT == kBF16 ? 2 : 4);
    static constexpr int bytes = vbytes + 16;
    static_assert(vbytes % 16 == 0, "row");
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ int valid_key(const MlaArgs& a, const int32_t* idxr, int j, int j_end, int L)
{
    const int s = j < j_end ? idxr[j] : -1;
    return (s >= 0 && s < L) ? s : -1;
}

// Units of consecutive index go to one XCD: blocks are dealt round-robin over
// the 8 XCDs, so block L runs on XCD L % 8.
__device__ __forceinline__ int xcd_unit(int L, int n_units)
{
    const int per = (n_units + 7) >> 3;
    return (L & 7) * per + (L >> 3);
}

// ================================================================ bf16 kernel
template <int DQK, int DV>
struct Bf16Cfg {
    static constexpr int ROWB = DQK * 2;          // bytes of a latent row
    static constexpr int CPR = DQK / 8;           // 16-byte chunks per row
    static constexpr int PCH = CPR + 1;           // LDS pitch in chunks (one pad chunk)
    static constexpr int PITCH = PCH * 16;
    static constexpr int TILE_CH = kTileKeys * PCH;
    static constexpr int DMA_PER_WAVE = (TILE_CH + 511) / 512;  // 1 KiB direct loads per wave per tile
    static constexpr int BUF_CH = DMA_PER_WAVE * 512;           // buffer size in chunks (dummy tail)
    static constexpr int NT = 512, NW = 8, DMA = DMA_PER_WAVE;   // for the asm gather
    static constexpr int HALF = DQK / 2;          // contraction share of a wave
    static constexpr int SHARE = DQK / 4;         // share of one 32-lane k-block
    static constexpr int QS = SHARE / 8;          // 32x32x16 steps over a half
    static constexpr int VH = DV / 2;             // value dims of a wave
    static constexpr int VT = VH / 32;            // 32-row value tiles of a wave
    static_assert(DQK % 32 == 0 && DV % 64 == 0 && DV <= DQK, "shape");
};

constexpr int kHeadsPerBlock = 128;  // 4 wave pairs x 32 heads
constexpr int kMaxListLen = 4096;    // longest index list a split holds in LDS

// Issue this wave's direct loads of index-list tile [j0, j0 + 32) into LDS
// buffer dst: position P holds row r = P / PCH, chunk P % PCH.  lrow holds the
// byte offset of each listed row from the sequence's base (row 0 for skipped
// entries, masked by the caller).  The pad chunk and the dummy tail past the
// tile fetch any row of the tile, so every wave issues exactly DMA_PER_WAVE
// loads.  Load k of a wave is position P0 + 512 k, so (r, chunk) advance by a
// constant step instead of a division per load.  All row offsets are read from
// LDS first, so the loads wait for one LDS round trip, not one per load.
template <class C>
__device__ __forceinline__ void gather_tile(const char* kvb, const uint32_t* lrow, int j0, int w, int lane,
                                            u32x4* dst)
{
    constexpr int DR = 512 / C::PCH, DCH = 512 % C::PCH;
    // an opaque lane id keeps the per-lane addresses out of the loop's live set
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wu = __builtin_amdgcn_readfirstlane(w);
    int r = (wu * 64 + ln) / C::PCH;
    int c = wu * 64 + ln - r * C::PCH;
    uint32_t roff[C::DMA_PER_WAVE], coff[C::DMA_PER_WAVE];
#pragma unroll
    for (int k = 0; k < C::DMA_PER_WAVE; ++k) {
        roff[k] = lrow[j0 + min(r, kTileKeys - 1)];
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

// Direct loads of index-list tile [j0, j0 + 32) into LDS, as gather_tile but for
// NT threads and issued from asm: gather_offsets reads the row offsets of this
// lane's DMA loads from LDS, gather_issue issues load k (M0 holds the wave's LDS
// destination).
template <class C>
__device__ __forceinline__ void gather_offsets(const uint32_t* lrow, int j0, int w, int lane, uint32_t (&off)[C::DMA])
{
    constexpr int DR = C::NT / C::PCH, DCH = C::NT % C::PCH;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wu = __builtin_amdgcn_readfirstlane(w);
    int r = (wu * 64 + ln) / C::PCH;
    int c = wu * 64 + ln - r * C::PCH;
#pragma unroll
    for (int k = 0; k < C::DMA; ++k) {
        off[k] = lrow[j0 + min(r, kTileKeys - 1)] + (c == C::CPR ? 0u : (uint32_t)c * 16u);
        r += DR;
        c += DCH;
        if (c >= C::PCH) {
            c -= C::PCH;
            ++r;
        }
    }
}

// STREAM marks the load non-temporal: for rows that no other query of the call
// reads (one query per sequence), so they do not displace cached data.
template <class C, bool STREAM = false>
__device__ __forceinline__ void gather_issue(const char* kvb, uint32_t off, u32x4* dst, int w, int k)
{
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) u32x4*)(dst + (wu + C::NW * k) * 64));
    if constexpr (STREAM)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(kvb), "{m0}"(lds) : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(kvb), "{m0}"(lds) : "memory");
}

// Direct loads of wave w that touch the tile (the others would fill only the
// dummy tail past it): the wave's loads k cover 64-chunk groups w + NW * k.
template <class C>
__device__ __forceinline__ int tile_loads(int w)
{
    constexpr int G = (C::TILE_CH + 63) / 64;
    return (G - w + C::NW - 1) / C::NW;
}

// SKIP_TAIL: leave out the loads that fill only the dummy tail; the caller's waits
// then count tile_loads(w) loads per tile for wave w.
template <class C, bool SKIP_TAIL = false, bool STREAM = false>
__device__ __forceinline__ void gather_tile_asm(const char* kvb, const uint32_t* lrow, int j0, int w, int lane,
                                                u32x4* dst)
{
    uint32_t off[C::DMA];
    gather_offsets<C>(lrow, j0, w, lane, off);
    const int n = SKIP_TAIL ? tile_loads<C>(__builtin_amdgcn_readfirstlane(w)) : C::DMA;
#pragma unroll
    for (int k = 0; k < C::DMA; ++k)
        if (k < n) gather_issue<C, STREAM>(kvb, off[k], dst, w, k);
}

// Workgroup barrier without the memory fence of __syncthreads (whose vmcnt(0)
// would also drain the tile prefetch): wait for this wave's LDS traffic (and,
// with VM, its direct loads), then s_barrier.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_lds_vm() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int DQK, int DV>
struct Bf16State {
    f32x16 o[Bf16Cfg<DQK, DV>::VT];
    float m_run, l_run;
};

// One 32-entry tile for wave (pair, half): partial S^T over the contraction
// half, exchange with the partner wave, online softmax, O^T[value half] += V^T.P^T.
template <int DQK, int DV>
__device__ __forceinline__ void tile_compute(const u32x4* tile, uint32_t vmask, const u32x4 (&qb)[Bf16Cfg<DQK, DV>::QS],
                                             Bf16State<DQK, DV>& st, float zc, float (*xbuf)[16][64], int w,
                                             int lane)
{
    using C = Bf16Cfg<DQK, DV>;
    asm volatile("" : "+v"(lane));  // lane-derived addresses are recomputed per tile, not kept live
    const int col = lane & 31, kb = lane >> 5, half = w & 1;
    const char* tb = reinterpret_cast<const char*>(tile);
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
    const char* kr = tb + col * C::PITCH + (C::HALF * half + C::SHARE * kb) * 2;
#pragma unroll
    for (int s = 0; s < C::QS; ++s) sacc = mfma32_bf16(*reinterpret_cast<const u32x4*>(kr + 16 * s), qb[s], sacc);
#pragma unroll
    for (int e = 0; e < 16; ++e) xbuf[w][e][lane] = sacc[e];
    barrier_lds();
    // lane holds keys 8*i + 4*kb + j (register 4*i + j) of head `col`; the
    // maximum is taken over q.k (zc > 0 keeps the order) and zc is folded into
    // the exponent below
    float tmax = -INFINITY;
    if (vmask == 0xFFFFFFFFu) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            sacc[e] += xbuf[w ^ 1][e][lane];
            tmax = fmaxf(tmax, sacc[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            const float sv = sacc[e] + xbuf[w ^ 1][e][lane];
            sacc[e] = ((vmask >> key) & 1u) ? sv : -INFINITY;
            tmax = fmaxf(tmax, sacc[e]);
        }
    }
    {
        // max with lane l ^ 32 on the gfx950 row swap (no LDS round trip)
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * zc;
    }
    // Lazy rescaling: the reference max m_run only moves when a logit exceeds
    // it by more than 8 (log2 units), so p <= 2^8 and O, l stay exact in fp32
    // while the rescale of O is rare.
    if (__ballot(tmax > st.m_run + 8.f)) {
        const float m_new = fmaxf(st.m_run, tmax);
        const float alpha = st.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int v = 0; v < C::VT; ++v) st.o[v] *= alpha;
        st.m_run = m_new;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        sacc[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], zc, -m_use));
        psum += sacc[e];
    }
    st.l_run += psum;
    // transpose-load roles: this lane supplies row 8*(2*step+i') + 4*kbv + jr, column vb + 4*qc
    const int grp = lane >> 4, m16 = lane & 15;
    const int kbv = grp >> 1, vb = 16 * (grp & 1);
    const int jr = m16 >> 2, qc = m16 & 3;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        u32x4 pb;
        pb[0] = pack_bf16x2(sacc[8 * step + 0], sacc[8 * step + 1]);
        pb[1] = pack_bf16x2(sacc[8 * step + 2], sacc[8 * step + 3]);
        pb[2] = pack_bf16x2(sacc[8 * step + 4], sacc[8 * step + 5]);
        pb[3] = pack_bf16x2(sacc[8 * step + 6], sacc[8 * step + 7]);
        const char* r0 = tb + (16 * step + 4 * kbv + jr) * C::PITCH + (C::VH * half + vb + 4 * qc) * 2;
        const char* r1 = r0 + 8 * C::PITCH;
#pragma unroll
        for (int v = 0; v < C::VT; ++v) {
            const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(r0 + 64 * v));
            const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(r1 + 64 * v));
            const u32x2 y0 = __builtin_bit_cast(u32x2, x0);
            const u32x2 y1 = __builtin_bit_cast(u32x2, x1);
            st.o[v] = mfma32_bf16(u32x4{y0[0], y0[1], y1[0], y1[1]}, pb, st.o[v]);
        }
    }
}

// Epilogue of the two-waves-per-SIMD fp8 kernel.  One row per head: the
// normalised value row in bf16 (the output row, or a split's partial row followed
// by its fp32 m, l).  Rows are staged in the free tile buffers and written out
// whole, 16 contiguous bytes per lane: two rounds of 64 heads, the pair p of a
// round staging its 32 rows in buffer p % 2.
template <int DQK, int DV, class C>
__device__ __forceinline__ void mla_write_rows(const MlaArgs& a, const Bf16State<DQK, DV>& st, u32x4* tA, u32x4* tB,
                                               int hb, size_t row, int rq, int split, int head, bool head_ok,
                                               int pair, int half, int col, int kb, int tid)
{
    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (a.n_split == 1 && a.lse && head_ok && half == 0 && kb == 0)
        a.lse[row * a.H + head] = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;

    using P = PartRow<kBF16, DV>;
    constexpr int SP = P::bytes;  // staged row pitch
    static_assert(32 * SP <= C::BUF_CH * 16, "staging rows");
    const bool part_out = a.n_split > 1;
    const int hb0 = hb * kHeadsPerBlock;
    const int heads_here = min(kHeadsPerBlock, a.H - hb0);
    char* gbase = part_out ? (char*)a.part + (((size_t)rq * a.n_split + split) * a.H + hb0) * P::bytes
                           : (char*)a.out + (row * a.H + hb0) * (size_t)(DV * 2);
    const int grow = part_out ? P::bytes : DV * 2;  // bytes of a row in global memory
    const int rch = grow / 16;
    barrier_lds();  // every wave is done reading the last tile
#pragma unroll 1
    for (int round = 0; round < 2; ++round) {
        if ((pair >> 1) == round) {
            // lane holds value dims VH*half + 32*v + 8*i + 4*kb + jj (register 4*i + jj) of head `col`
            char* sb = reinterpret_cast<char*>((pair & 1) ? tB : tA) + col * SP + (C::VH * half + 4 * kb) * 2;
#pragma unroll
            for (int v = 0; v < C::VT; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 w2 = {pack_bf16x2(st.o[v][4 * i] * inv, st.o[v][4 * i + 1] * inv),
                                      pack_bf16x2(st.o[v][4 * i + 2] * inv, st.o[v][4 * i + 3] * inv)};
                    *reinterpret_cast<u32x2*>(sb + 2 * (32 * v + 8 * i)) = w2;
                }
            if (half == 0 && kb == 0)
                *reinterpret_cast<f32x4*>(reinterpret_cast<char*>((pair & 1) ? tB : tA) + col * SP + P::vbytes) =
                    f32x4{st.m_run, l_tot, 0.f, 0.f};
        }
        barrier_lds();
        const int h0 = 64 * round;
        const int n = min(64, heads_here - h0) * rch;
        for (int c = tid; c < n; c += 512) {
            const int r = c / rch, k = c - r * rch;
            const char* sb = reinterpret_cast<const char*>((r >> 5) ? tB : tA) + (r & 31) * SP + 16 * k;
            st16(gbase + (size_t)(h0 + r) * grow + 16 * k, *reinterpret_cast<const u32x4*>(sb));
        }
        if (round == 0) barrier_lds();
    }
}

// Epilogue of the bf16 kernels, staged through LDS: a workgroup's rows (one per
// head: the normalised value row in bf16, or a split's partial row followed by its
// fp32 m, l) are one contiguous block in memory, so each wave first writes its
// share into `stage` (row pitch PartRow::bytes, conflict-free for the 8-byte
// writes) and the whole block then leaves in 1 KiB stores.  The caller's lane holds
// value dims d0 + 32*v + 8*i + 4*kb + jj (register 4*i + jj) of staging row `srow`
// (head hb * 128 + srow); `ml` marks the one lane per row that writes m and l;
// `l_tot` is the row's softmax sum.  The block is written once (and partials read
// once, by the combine), so the stores carry the non-temporal hint.
template <int DV, int VT, int NT>
__device__ __forceinline__ void mla_write_rows_staged(const MlaArgs& a, const f32x16 (&o)[VT], float m_run,
                                                      float l_tot, size_t row, int rq, int split, int hb, int srow,
                                                      int d0, int kb, bool ml, int tid, char* stage)
{
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    using P = PartRow<kBF16, DV>;
    constexpr int SP = P::bytes;  // staged row pitch
    const bool part_out = a.n_split > 1;
    const int hb0 = hb * kHeadsPerBlock;
    const int heads_here = min(kHeadsPerBlock, a.H - hb0);
    char* gbase = part_out ? (char*)a.part + (((size_t)rq * a.n_split + split) * a.H + hb0) * P::bytes
                           : (char*)a.out + (row * a.H + hb0) * (size_t)(DV * 2);
    const int rch = part_out ? P::bytes / 16 : DV / 8;  // 16-byte chunks of a row in memory
    barrier_lds();  // every wave is done with the tiles (and any flags read after the loop)
    char* sb = stage + srow * SP + 2 * d0 + 8 * kb;
#pragma unroll
    for (int v = 0; v < VT; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x2*>(sb + 2 * (32 * v + 8 * i)) =
                u32x2{pack_bf16x2(o[v][4 * i] * inv, o[v][4 * i + 1] * inv),
                      pack_bf16x2(o[v][4 * i + 2] * inv, o[v][4 * i + 3] * inv)};
    if (ml) *reinterpret_cast<f32x4*>(stage + srow * SP + P::vbytes) = f32x4{m_run, l_tot, 0.f, 0.f};
    barrier_lds();
    const int n = heads_here * rch;
    for (int c = tid; c < n; c += NT) {
        const int r = c / rch, k = c - r * rch;
        st16_nt(gbase + 16 * (size_t)c, *reinterpret_cast<const u32x4*>(stage + r * SP + 16 * k));
    }
}

// One 512-thread workgroup (8 waves, two per SIMD) owns a (query, split of the
// index list) unit and 128 heads.  Wave w = (pair w/2, half w%2): heads
// 32*(w/2).., contraction half and value half w%2.  Two LDS tile buffers named
// statically (loop unrolled by two) keep the next tile's gather in flight
// while the current one is consumed.
template <int DQK, int DV>
__global__ __launch_bounds__(512) void mla_bf16_kernel(MlaArgs a)
{
    using C = Bf16Cfg<DQK, DV>;
    // the queries of wave pair p are staged in region p (see the prologue), which
    // overlays the tile buffers, the logit exchange and the index list
    constexpr int kStageCh = (kTileKeys * C::PCH + 63) / 64 * 64;  // one pair's 32 padded rows
    constexpr int kStageLoads = kStageCh / 64;
    constexpr int kXbufCh = 8 * 16 * 64 / 4;
    constexpr int kListWords = kMaxListLen + kMaxListLen / kTileKeys;
    constexpr int kMainCh = 2 * C::BUF_CH + kXbufCh + (kListWords + 3) / 4;
    constexpr int kLdsCh = 4 * kStageCh > kMainCh ? 4 * kStageCh : kMainCh;
    __shared__ __attribute__((aligned(16))) u32x4 lds[kLdsCh];
    u32x4* tA = lds;
    u32x4* tB = lds + C::BUF_CH;
    float (*xbuf)[16][64] = reinterpret_cast<float (*)[16][64]>(lds + 2 * C::BUF_CH);
    uint32_t* lrow = reinterpret_cast<uint32_t*>(lds + 2 * C::BUF_CH + kXbufCh);
    uint32_t* tmask = lrow + kMaxListLen;

    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int n_units = a.B * a.t_count * a.n_split * HB;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int hb = unit % HB;
    const int split = (unit / HB) % a.n_split;
    const int rq = unit / HB / a.n_split;
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;
    const int L = min(a.kv_len[b], a.Lmax);

    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int pair = w >> 1, half = w & 1;
    const int col = lane & 31, kb = lane >> 5;
    const int head = hb * kHeadsPerBlock + pair * 32 + col;
    const bool head_ok = head < a.H;

    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);
    // an empty sequence (L = 0) has no row to gather, not even the stand-in row 0
    const int n_tiles = (j_end > j_begin && L > 0) ? (j_end - j_begin + kTileKeys - 1) / kTileKeys : 0;

    const char* kvb = (const char*)a.kv + (size_t)b * a.Lmax * C::ROWB;
    const int32_t* idxr = a.idx + row * a.K;
    // The split's index list is loaded first and Q behind it: loads complete in
    // order, so waiting for the list leaves the Q loads in flight through the list
    // set-up and the first gather.
    // (unconditional loads, clamped into the list: a load under a branch would make
    // the compiler wait for every load at the join)
    constexpr int kListPer = kMaxListLen / 512;
    const int n_list = n_tiles * kTileKeys;
    const int j_last = max(j_end - 1, 0);
    int raw[kListPer];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) raw[r] = idxr[min(j_begin + tid + 512 * r, j_last)];
    // Q^T operand: head `head`, contraction d in [HALF*half + SHARE*kb, + SHARE).  The
    // pair's 32 query rows are contiguous in memory and are staged in LDS by direct
    // 1 KiB loads in the tiles' padded layout (position P: row P / PCH, chunk P % PCH,
    // the pad chunk a copy of chunk 0; half h of the pair issues loads h, h + 2, ...).
    // A row past the last head reads head H - 1 (finite values whose results are never
    // written), so every load is unconditional.
    {
        const char* qbase = (const char*)a.q + row * (size_t)a.H * C::ROWB;
        const int pu = __builtin_amdgcn_readfirstlane(pair), hu = __builtin_amdgcn_readfirstlane(half);
        const int h0 = hb * kHeadsPerBlock + pu * 32;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int hr = 0, ch = ln + 64 * hu;  // position of load hu: 64 hu + lane
        while (ch >= C::PCH) {
            ch -= C::PCH;
            ++hr;
        }
#pragma unroll
        for (int k = 0; k < (kStageLoads + 1) / 2; ++k) {
            const int kk = 2 * k + hu;
            if (kk < kStageLoads) {
                const int hh = min(h0 + min(hr, kTileKeys - 1), a.H - 1);
                const uint32_t off = (uint32_t)hh * C::ROWB + (ch >= C::CPR ? 0u : (uint32_t)ch * 16u);
                const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(
                    (__attribute__((address_space(3))) u32x4*)(lds + pu * kStageCh + 64 * kk));
                asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(qbase), "{m0}"(dst)
                             : "memory");
            }
            ch += 128;  // two loads further on
            while (ch >= C::PCH) {
                ch -= C::PCH;
                ++hr;
            }
        }
    }
    barrier_lds_vm();  // the pair's staged queries have landed
    u32x4 qb[C::QS];
    {
        const char* qr = reinterpret_cast<const char*>(lds + pair * kStageCh) + col * C::PITCH +
                         (C::HALF * half + C::SHARE * kb) * 2;
#pragma unroll
        for (int s = 0; s < C::QS; ++s) qb[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
    }
    barrier_lds();  // every wave has its queries: the staging area is free
    // the list sanitised (skipped entries fetch row 0) and padded to whole tiles,
    // plus a validity mask per tile; every slot is filled (the ones past the list
    // as skipped), without branches, so the compiler keeps the early loads
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
        const int j = tid + 512 * r;
        const int s = raw[r];
        const bool ok = j < n_list && j_begin + j < j_end && s >= 0 && s < L;
        lrow[j] = ok ? (uint32_t)s * C::ROWB : 0u;
        const uint64_t bits = __ballot(ok);  // 64 consecutive entries = two tiles
        if (lane == 0) {  // j is a multiple of 64 here, so both words lie inside tmask
            tmask[j / kTileKeys] = (uint32_t)bits;
            tmask[j / kTileKeys + 1] = (uint32_t)(bits >> 32);
        }
    }
    barrier_lds();

    Bf16State<DQK, DV> st;
#pragma unroll
    for (int v = 0; v < C::VT; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    const float zc = a.sm_scale * kLog2e;

    // tile `it` lives in buffer it % 2; each step issues tile it + 1 into the other buffer
    if (n_tiles > 0) gather_tile_asm<C, true>(kvb, lrow, 0, w, lane, tA);
#pragma unroll 1
    for (int it = 0; it < n_tiles; it += 2) {
        barrier_lds_vm();
        // the tile's mask is read together with the next tile's row offsets
        const uint32_t vmA = tmask[it];
        if (it + 1 < n_tiles) gather_tile_asm<C, true>(kvb, lrow, (it + 1) * kTileKeys, w, lane, tB);
        __builtin_amdgcn_sched_barrier(0);
        tile_compute<DQK, DV>(tA, vmA, qb, st, zc, xbuf, w, lane);
        if (it + 1 >= n_tiles) break;
        barrier_lds_vm();
        const uint32_t vmB = tmask[it + 1];
        if (it + 2 < n_tiles) gather_tile_asm<C, true>(kvb, lrow, (it + 2) * kTileKeys, w, lane, tA);
        __builtin_amdgcn_sched_barrier(0);
        tile_compute<DQK, DV>(tB, vmB, qb, st, zc, xbuf, w, lane);
    }

    static_assert(kHeadsPerBlock * PartRow<kBF16, DV>::bytes <= (int)sizeof(lds), "output staging");
    {
        const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
        if (a.n_split == 1 && a.lse && head_ok && half == 0 && kb == 0)
            a.lse[row * a.H + head] = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        mla_write_rows_staged<DV, C::VT, C::NT>(a, st.o, st.m_run, l_tot, row, rq, split, hb, pair * 32 + col,
                                                C::VH * half, kb, half == 0 && kb == 0, tid,
                                                reinterpret_cast<char*>(lds));
    }
}

// ================================================================ wide bf16 kernel
// One 256-thread workgroup (four waves, one per SIMD) per (query, split, 128
// heads).  Wave w owns heads 32w .. 32w + 31 over the whole contraction and the
// whole value row: no logits are exchanged between waves and no softmax is
// computed twice.  With one wave per SIMD the softmax's VALU work issues
// beside the MFMAs of the same wave (a 32x32x16 MFMA hides about four VALU
// instructions there, while at two waves per SIMD with VGPR accumulators the
// two add up).  The value accumulators (DV x 32 heads per wave) take the
// accumulation registers.  Three LDS tile buffers keep two gathers in flight.
// The gathers are issued from inline asm, so the compiler's tracking of direct
// LDS loads cannot turn them into a full wait before every LDS read; the waits
// on them are explicit (vmcnt counts a wave's loads in issue order).
template <int DQK, int DV>
struct WideCfg {
    static constexpr int NT = 256;                 // threads per workgroup
    static constexpr int NW = NT / 64;
    static constexpr int ROWB = DQK * 2;
    static constexpr int CPR = DQK / 8;
    static constexpr int PCH = CPR + 1;            // odd pitch in chunks: conflict-free 16-byte columns
    static constexpr int PITCH = PCH * 16;
    static constexpr int TILE_CH = kTileKeys * PCH;
    static constexpr int DMA = (TILE_CH + NT - 1) / NT;  // direct loads per wave per tile
    static constexpr int BUF_CH = DMA * NT;
    static constexpr int NBUF = 3;
    static constexpr int QS = DQK / 16;            // 32x32x16 steps over the contraction
    static constexpr int HQ = DQK / 2;             // contraction share of a lane half
    static constexpr int VT = DV / 32;             // 32-row value tiles
    static constexpr int K_AHEAD = 4;              // key reads in flight ahead of the logit MFMAs
    static constexpr int V_AHEAD = 4;              // value reads in flight ahead of the value MFMAs
    static_assert(DQK % 32 == 0 && DV % 32 == 0 && DV <= DQK, "shape");
};

// The logits' 32x32x16 bf16 MFMAs, written as asm so that their accumulator stays
// in VGPRs (the softmax reads it) while the compiler gives the value
// accumulators every AGPR; left to itself it puts both in AGPRs and spills.
// The compiler does not see these as MFMAs: wait_mfma_acc() covers the hazard
// before other instructions read the result.
__device__ __forceinline__ void mfma32_bf16_vfirst(u32x4 a, u32x4 b, f32x16& acc)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_bf16_vacc(u32x4 a, u32x4 b, f32x16& acc)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 18 wait states: more than a 32x32x16 MFMA's result needs before other
// instructions may read its destination.  Taking the result as an operand keeps
// every later reader after the wait.
__device__ __forceinline__ void wait_mfma_acc(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+v"(x)); }

// The wide kernel's softmax keeps a per-head reference m (log2 domain) instead
// of the running maximum: p = 2^(z - m) stays below 2^kWideSlack, far inside
// fp32 and bf16 range.  A logit more than kWideSlack above m (never on the
// first valid tile, which sets m) restarts the unit from its first tile with
// the raised reference, so the value accumulators are never rescaled by VALU
// code inside the tile loop, which would make the compiler move them out of
// the AGPRs on every iteration.
constexpr float kWideSlack = 64.f;

template <int DQK, int DV>
struct WideState {
    f32x16 o[WideCfg<DQK, DV>::VT];
    float m_run, l_run;
};

// A gather carried out by the tile computation: its loads are issued one at a
// time between the logit MFMAs, so that they queue behind no other wave's burst
// and the wave keeps issuing MFMAs meanwhile.  Load k's row offset is read from
// LDS a few MFMAs before it is issued; (r, c) step through this lane's
// positions as in gather_offsets.
template <class C>
struct PendingGather {
    const char* kvb;
    u32x4* dst;
    const uint32_t* lrow;  // entry j0 of the tile's list
    int r, c;
    bool active;
    __device__ __forceinline__ void start(int w, int lane)
    {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int wu = __builtin_amdgcn_readfirstlane(w);
        r = (wu * 64 + ln) / C::PCH;
        c = wu * 64 + ln - r * C::PCH;
    }
    __device__ __forceinline__ uint32_t next_offset()
    {
        constexpr int DR = C::NT / C::PCH, DCH = C::NT % C::PCH;
        const uint32_t off = lrow[min(r, kTileKeys - 1)] + (c == C::CPR ? 0u : (uint32_t)c * 16u);
        r += DR;
        c += DCH;
        if (c >= C::PCH) {
            c -= C::PCH;
            ++r;
        }
        return off;
    }
};

// Wait until at most N direct loads of this wave are outstanding and its LDS
// traffic is done, then s_barrier.
template <int N>
__device__ __forceinline__ void barrier_vm()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// One 32-key tile for one wave: S^T[32 keys x 32 heads] = K . Q^T over the whole
// contraction, online softmax, O^T[DV x 32 heads] += V^T . P^T.  The LDS reads
// feeding the MFMAs go in groups of four steps, the next group's reads issued
// before the current group's MFMAs, with a scheduling barrier between groups:
// without it the compiler hoists every read of the tile and spills the queries.
template <int DQK, int DV, bool STREAM>
__device__ __forceinline__ bool tile_compute_wide(const u32x4* tile, uint32_t vmask,
                                                  const u32x4 (&qb)[WideCfg<DQK, DV>::QS], WideState<DQK, DV>& st,
                                                  float zc, int lane, int w, PendingGather<WideCfg<DQK, DV>>& pg)
{
    using C = WideCfg<DQK, DV>;
    constexpr int GAP = C::QS / C::DMA;  // logit steps between two loads of the pending gather
    static_assert(GAP >= 1, "gather spacing");
    constexpr int DK = C::K_AHEAD, DVW = C::V_AHEAD;
    asm volatile("" : "+v"(lane));
    const int col = lane & 31, kb = lane >> 5;
    const char* tb = reinterpret_cast<const char*>(tile);
    f32x16 sacc;
    const char* kr = tb + col * C::PITCH + C::HQ * kb * 2;
    {
        // rolling window: the read for step s + DK is issued before the MFMA of step s
        uint32_t goff = 0;
        u32x4 kw[DK];
#pragma unroll
        for (int j = 0; j < DK; ++j) kw[j] = *reinterpret_cast<const u32x4*>(kr + 16 * j);
#pragma unroll
        for (int st_ = 0; st_ < C::QS; ++st_) {
            const u32x4 ka = kw[st_ % DK];
            if (st_ + DK < C::QS) kw[st_ % DK] = *reinterpret_cast<const u32x4*>(kr + 16 * (st_ + DK));
            if (st_ == 0)
                mfma32_bf16_vfirst(ka, qb[0], sacc);
            else
                mfma32_bf16_vacc(ka, qb[st_], sacc);
            if (st_ % GAP == 0 && st_ / GAP < C::DMA) goff = pg.next_offset();
            if (st_ % GAP == GAP - 1 && st_ / GAP < C::DMA && pg.active)
                gather_issue<C, STREAM>(pg.kvb, goff, pg.dst, w, st_ / GAP);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_mfma_acc(sacc);
    // lane holds keys 8*i + 4*kb + j (register 4*i + j) of head `col`
    float tmax = -INFINITY;
    if (vmask == 0xFFFFFFFFu) {
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            sacc[e] = ((vmask >> key) & 1u) ? sacc[e] : -INFINITY;
            tmax = fmaxf(tmax, sacc[e]);
        }
    }
    {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * zc;
    }
    if (__ballot(tmax > st.m_run + kWideSlack)) {
        // a head with no valid key so far takes this tile's maximum (its sums are
        // zero); a head whose reference is exceeded by more than the slack needs
        // a restart, and this tile's value sum is skipped
        const bool over = __ballot(st.m_run != -INFINITY && tmax > st.m_run + kWideSlack) != 0;
        if (tmax > st.m_run + kWideSlack) st.m_run = tmax;
        if (over) return true;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        sacc[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], zc, -m_use));
        psum += sacc[e];
    }
    st.l_run += psum;
    // transpose-load roles: this lane supplies row 8*(2*step+i') + 4*kbv + jr, column vb + 4*qc
    const int grp = lane >> 4, m16 = lane & 15;
    const int kbv = grp >> 1, vb = 16 * (grp & 1);
    const int jr = m16 >> 2, qc = m16 & 3;
    const char* r0 = tb + (4 * kbv + jr) * C::PITCH + (vb + 4 * qc) * 2;
    u32x4 pb[2];
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        pb[step][0] = pack_bf16x2(sacc[8 * step + 0], sacc[8 * step + 1]);
        pb[step][1] = pack_bf16x2(sacc[8 * step + 2], sacc[8 * step + 3]);
        pb[step][2] = pack_bf16x2(sacc[8 * step + 4], sacc[8 * step + 5]);
        pb[step][3] = pack_bf16x2(sacc[8 * step + 6], sacc[8 * step + 7]);
    }
    // MFMA n = step * VT + v reads rows 16*step + (0 | 8) + ..., columns 32*v + ...
    auto ld_pair = [&](int n, u32x4& x) {
        const int step = n / C::VT, v = n % C::VT;
        const char* p0 = r0 + 16 * step * C::PITCH + 64 * v;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p0 + 8 * C::PITCH));
        const u32x2 y0 = __builtin_bit_cast(u32x2, x0);
        const u32x2 y1 = __builtin_bit_cast(u32x2, x1);
        x = u32x4{y0[0], y0[1], y1[0], y1[1]};
    };
    constexpr int NPV = 2 * C::VT;
    u32x4 vw[DVW];
#pragma unroll
    for (int j = 0; j < DVW; ++j) ld_pair(j, vw[j]);
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
        const u32x4 va = vw[n % DVW];
        if (n + DVW < NPV) ld_pair(n + DVW, vw[n % DVW]);
        st.o[n % C::VT] = mfma32_bf16(va, pb[n / C::VT], st.o[n % C::VT]);
        __builtin_amdgcn_sched_barrier(0);
    }
    return false;
}

// Epilogue of the wide kernels: one row per head (the normalised value row in
// bf16, or a split's partial row followed by its fp32 m, l), stored straight from
// registers.  A lane holds dims 32*v + 8*i + 4*kb + jj (register 4*i + jj) of
// head `col`; trading half of them with lane ^ 32 leaves lane (col, 0) with dims
// 32*v + [0, 8) and + [16, 24), lane (col, 1) with + [8, 16) and + [24, 32), so
// every store is 16 contiguous bytes.
template <int DQK, int DV, class C>
__device__ __forceinline__ void mla_write_rows_wide(const MlaArgs& a, const WideState<DQK, DV>& st, size_t row,
                                                    int rq, int split, int head, bool head_ok, int kb)
{
    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (a.n_split == 1 && a.lse && head_ok && kb == 0)
        a.lse[row * a.H + head] = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    using P = PartRow<kBF16, DV>;
    const bool part_out = a.n_split > 1;
    const size_t hrow = head_ok ? (size_t)head : 0;
    char* rowp = part_out ? (char*)a.part + (((size_t)rq * a.n_split + split) * a.H + hrow) * P::bytes
                          : (char*)a.out + (row * a.H + hrow) * (size_t)(DV * 2);
#pragma unroll
    for (int v = 0; v < C::VT; ++v) {
        uint32_t d[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = pack_bf16x2(st.o[v][4 * i] * inv, st.o[v][4 * i + 1] * inv);
            d[2 * i + 1] = pack_bf16x2(st.o[v][4 * i + 2] * inv, st.o[v][4 * i + 3] * inv);
        }
#pragma unroll
        for (int x = 0; x < 8; x += 4)
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                const uint32_t send = kb ? d[x + y] : d[x + y + 2];
                const uint32_t got = (uint32_t)__shfl_xor((int)send, 32, 64);
                if (kb)
                    d[x + y] = got;
                else
                    d[x + y + 2] = got;
            }
        if (head_ok) {
            st16(rowp + 2 * (32 * v + 8 * kb), u32x4{d[0], d[1], d[2], d[3]});
            st16(rowp + 2 * (32 * v + 16 + 8 * kb), u32x4{d[4], d[5], d[6], d[7]});
        }
    }
    if (part_out && head_ok && kb == 0)
        *reinterpret_cast<f32x4*>(rowp + P::vbytes) = f32x4{st.m_run, l_tot, 0.f, 0.f};
}

// Queries of the wide kernel staged through LDS: wave w's 32 query rows are
// contiguous in memory, so they are loaded 1 KiB per instruction straight into
// LDS in the tiles' padded layout (32 rows of PCH chunks, the pad chunk a copy of
// chunk 0), and each lane then reads its MFMA operand the way it reads the keys.
// The staging area overlays the tile buffers and the index list, which are
// filled only after every wave has read its queries.
template <class C>
struct WideQStage {
    static constexpr int ROW_CH = kTileKeys * C::PCH;                   // 32 rows, padded pitch
    static constexpr int LOADS = (ROW_CH + 63) / 64;                    // 1 KiB loads per wave
    static constexpr int WAVE_CH = LOADS * 64;                          // a wave's staging chunks
    static constexpr int CH = C::NW * WAVE_CH;
};

template <int DQK, int DV, bool STREAM>
__global__ __launch_bounds__(256) void mla_wide_kernel(MlaArgs a)
{
    using C = WideCfg<DQK, DV>;
    using QS_ = WideQStage<C>;
    constexpr int kTileCh = C::NBUF * C::BUF_CH;
    constexpr int kListWords = kMaxListLen + kMaxListLen / kTileKeys + 2;
    constexpr int kMainCh = kTileCh + (kListWords + 3) / 4;
    __shared__ __attribute__((aligned(16))) u32x4 lds[QS_::CH > kMainCh ? QS_::CH : kMainCh];
    u32x4* tiles = lds;
    uint32_t* lrow = reinterpret_cast<uint32_t*>(lds + kTileCh);
    uint32_t* tmask = lrow + kMaxListLen;
    // restart requests: a wave raising one during tile `it` writes slot it & 1,
    // which every wave reads after the next barrier (before anyone can write that
    // slot again, two tiles later)
    volatile int* restart = reinterpret_cast<volatile int*>(tmask + kMaxListLen / kTileKeys);

    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int n_units = a.B * a.t_count * a.n_split * HB;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int hb = unit % HB;
    const int split = (unit / HB) % a.n_split;
    const int rq = unit / HB / a.n_split;
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;
    const int L = min(a.kv_len[b], a.Lmax);

    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int col = lane & 31, kb = lane >> 5;
    const int head = hb * kHeadsPerBlock + w * 32 + col;
    const bool head_ok = head < a.H;

    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);
    // an empty sequence (L = 0) has no row to gather, not even the stand-in row 0
    const int n_tiles = (j_end > j_begin && L > 0) ? (j_end - j_begin + kTileKeys - 1) / kTileKeys : 0;

    const char* kvb = (const char*)a.kv + (size_t)b * a.Lmax * C::ROWB;
    const int32_t* idxr = a.idx + row * a.K;
    constexpr int kListPer = kMaxListLen / C::NT;
    const int n_list = n_tiles * kTileKeys;
    const int j_last = max(j_end - 1, 0);
    int raw[kListPer];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) raw[r] = idxr[min(j_begin + tid + C::NT * r, j_last)];
    // Q^T operand: lane (col, kb) holds dims [HQ * kb + 8 s, + 8) of head `col` at step s.
    // Staging position p of wave w is row p / PCH (head 32 w + p / PCH, rows past the
    // wave's 32 and heads past H read head H - 1), chunk p % PCH (the pad chunk reads
    // chunk 0); load k covers positions 64 k .. 64 k + 63.
    {
        const char* qbase = (const char*)a.q + row * (size_t)a.H * C::ROWB;
        const int wu = __builtin_amdgcn_readfirstlane(w);
        const int h0 = hb * kHeadsPerBlock + wu * 32;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int hr = 0, ch = ln;  // position of load 0: lane
        while (ch >= C::PCH) {
            ch -= C::PCH;
            ++hr;
        }
#pragma unroll
        for (int k = 0; k < QS_::LOADS; ++k) {
            const int hh = min(h0 + min(hr, kTileKeys - 1), a.H - 1);
            const uint32_t off = (uint32_t)hh * C::ROWB + (ch >= C::CPR ? 0u : (uint32_t)ch * 16u);
            const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) u32x4*)(lds + wu * QS_::WAVE_CH + 64 * k));
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(qbase), "{m0}"(dst)
                         : "memory");
            ch += 64;
            while (ch >= C::PCH) {
                ch -= C::PCH;
                ++hr;
            }
        }
    }
    barrier_lds_vm();  // this wave's staged queries have landed (and everyone's)
    u32x4 qb[C::QS];
    {
        const char* qr = reinterpret_cast<const char*>(lds + w * QS_::WAVE_CH) + col * C::PITCH + C::HQ * kb * 2;
#pragma unroll
        for (int s = 0; s < C::QS; ++s) qb[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
    }
    barrier_lds();  // every wave has its queries: the staging area is free
    if (tid < 2) restart[tid] = 0;
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
        const int j = tid + C::NT * r;
        const int s = raw[r];
        const bool ok = j < n_list && j_begin + j < j_end && s >= 0 && s < L;
        lrow[j] = ok ? (uint32_t)s * C::ROWB : 0u;
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {  // j is a multiple of 64 here, so both words lie inside tmask
            tmask[j / kTileKeys] = (uint32_t)bits;
            tmask[j / kTileKeys + 1] = (uint32_t)(bits >> 32);
        }
    }
    // the queries have arrived before the first gather is issued (the waits the
    // compiler places for them cannot see the asm loads and would drain those too)
#pragma unroll
    for (int s = 0; s < C::QS; ++s) asm volatile("" : "+v"(qb[s]));
    barrier_lds();

    WideState<DQK, DV> st;
#pragma unroll
    for (int v = 0; v < C::VT; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    const float zc = a.sm_scale * kLog2e;

#pragma unroll 1
    for (;;) {
        if (n_tiles > 0) gather_tile_asm<C, false, STREAM>(kvb, lrow, 0, w, lane, tiles);
        if (n_tiles > 1) gather_tile_asm<C, false, STREAM>(kvb, lrow, kTileKeys, w, lane, tiles + C::BUF_CH);
        int cur = 0;
#pragma unroll 1
        for (int it = 0; it < n_tiles; ++it) {
            // tile `it` has landed everywhere and every wave is done with the buffer
            // it computed two tiles ago, which the gather below refills (a wave's
            // loads retire in order: at most the next tile's may still be in flight)
            if (it + 1 < n_tiles)
                barrier_vm<C::DMA>();
            else
                barrier_vm<0>();
            if (it > 0 && restart[(it - 1) & 1]) break;  // read after the barrier: the same for every wave
            const uint32_t vm = tmask[it];
            const int nxt = cur == 0 ? 2 : cur - 1;  // (cur + 2) % 3
            PendingGather<C> pg;
            pg.kvb = kvb;
            pg.dst = tiles + nxt * C::BUF_CH;
            pg.lrow = lrow + min(it + 2, n_tiles - 1) * kTileKeys;
            pg.active = it + 2 < n_tiles;
            pg.start(w, lane);
            if (tile_compute_wide<DQK, DV, STREAM>(tiles + cur * C::BUF_CH, vm, qb, st, zc, lane, w, pg) && lane == 0)
                restart[it & 1] = 1;
            cur = cur == 2 ? 0 : cur + 1;
        }
        barrier_vm<0>();  // no gather in flight, every flag write visible
        if (!(restart[0] | restart[1])) break;
        // a reference was raised: start the unit over (the references are kept)
        barrier_lds();
        if (tid < 2) restart[tid] = 0;
#pragma unroll
        for (int v = 0; v < C::VT; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
        st.l_run = 0.f;
    }
    static_assert(kHeadsPerBlock * PartRow<kBF16, DV>::bytes <= (int)sizeof(lds), "output staging");
    if (a.n_split > 1) {
        // split partials (decode): staged through LDS, written in 1 KiB stores
        const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
        mla_write_rows_staged<DV, C::VT, C::NT>(a, st.o, st.m_run, l_tot, row, rq, split, hb, w * 32 + col, 0, kb,
                                                kb == 0, tid, reinterpret_cast<char*>(lds));
    } else {
        // output rows (prefill): stored from registers; staged, the full causal
        // prefill_32k MLA measured 1% slower
        mla_write_rows_wide<DQK, DV, C>(a, st, row, rq, split, head, head_ok, kb);
    }
}

// ================================================================ wide fp8 kernel
// The wide kernel on the fp8 latent cache: a row is 576 e4m3 codes and its
// scale chunk (592 bytes), q arrives as codes with one scale per (query, head).
// Per 32-key tile a wave reads half the LDS bytes of the bf16 kernel: q.k runs on
// the 32x32x64 f8f6f4 MFMA (two 16-byte reads per 64-deep step), and the value
// operand comes from one 8-bit transpose read per MFMA, converted to bf16 by
// v_cvt_scalef32_pk_bf16_fp8 (scale 1: exact, e4m3 has three mantissa bits).
template <int DQK, int DV>
struct Fp8WideCfg {
    static constexpr int NT = 256;
    static constexpr int NW = NT / 64;
    static constexpr int ROWB = DQK + 16;          // codes + scale chunk
    static constexpr int CPR = ROWB / 16;
    static constexpr int PCH = CPR;                // odd pitch in chunks
    static constexpr int PITCH = PCH * 16;
    static constexpr int TILE_CH = kTileKeys * PCH;
    static constexpr int DMA = (TILE_CH + NT - 1) / NT;
    static constexpr int BUF_CH = DMA * NT;
    static constexpr int NBUF = 4;                 // three gathers in flight; room to stage 64 output rows
    static constexpr int QS = DQK / 64;            // 32x32x64 steps
    static constexpr int VT = DV / 32;
    static constexpr int V_AHEAD = 4;              // value reads in flight ahead of the value MFMAs
    static_assert(DQK % 64 == 0 && DV % 32 == 0 && DV <= DQK && CPR % 2 == 1, "shape");
};

// f8f6f4 32x32x64 MFMA (both operands e4m3, unit block scales in `one` = 127)
// accumulating in VGPRs, as asm for the same reason as the bf16 logits.
__device__ __forceinline__ void mfma32_fp8_vfirst(const i32x8& a, const i32x8& b, int one, f32x16& acc)
{
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
                 : "=&v"(acc) : "v"(a), "v"(b), "v"(one));
}
__device__ __forceinline__ void mfma32_fp8_vacc(const i32x8& a, const i32x8& b, int one, f32x16& acc)
{
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(acc) : "v"(a), "v"(b), "v"(one));
}
// 24 wait states: more than the 16-pass f8f6f4 MFMA's result needs.
__device__ __forceinline__ void wait_mfma16_acc(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x)); }

template <int DQK, int DV>
__device__ __forceinline__ bool tile_compute_fp8w(const u32x4* tile, uint32_t vmask,
                                                  const i32x8 (&qb)[Fp8WideCfg<DQK, DV>::QS], WideState<DQK, DV>& st,
                                                  float zch, int lane, int w, float* kscol,
                                                  PendingGather<Fp8WideCfg<DQK, DV>>& pg)
{
    using C = Fp8WideCfg<DQK, DV>;
    asm volatile("" : "+v"(lane));
    const int col = lane & 31, kb = lane >> 5;
    const char* tb = reinterpret_cast<const char*>(tile);
    // key scales: lane l reads key l % 32's scale into this wave's column, then
    // takes keys 8*i + 4*kb .. + 3 with one 16-byte read per i
    const float ksl = *reinterpret_cast<const float*>(tb + col * C::PITCH + DQK);
    if (kb == 0) kscol[col] = ksl;
    f32x16 sacc;
    const int one = 127;
    const char* kr = tb + col * C::PITCH + 32 * kb;
    {
        constexpr int GAP = (C::QS * 2) / C::DMA;  // half-steps between gather loads
        static_assert(GAP >= 2, "gather spacing");
        uint32_t goff = 0;
        i32x8 kw[2];
        auto ldk = [&](int s) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + 64 * s);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + 64 * s + 16);
            return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        kw[0] = ldk(0);
        kw[1] = ldk(1);
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
            const i32x8 ka = kw[s & 1];
            if (s + 2 < C::QS) kw[s & 1] = ldk(s + 2);
            if (s == 0)
                mfma32_fp8_vfirst(ka, qb[0], one, sacc);
            else
                mfma32_fp8_vacc(ka, qb[s], one, sacc);
            // the pending gather: load k's row offset is read at half-step GAP * k
            // and the load issued at half-step GAP * k + GAP - 1
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hs = 2 * s + h;
                if (hs % GAP == 0 && hs / GAP < C::DMA) goff = pg.next_offset();
                if (hs % GAP == GAP - 1 && hs / GAP < C::DMA && pg.active)
                    gather_issue<C>(pg.kvb, goff, pg.dst, w, hs / GAP);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_mfma16_acc(sacc);
    float ks[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(kscol + 8 * i + 4 * kb);
#pragma unroll
        for (int j = 0; j < 4; ++j) ks[4 * i + j] = k4[j];
    }
    // lane holds keys 8*i + 4*kb + j (register 4*i + j) of head `col`
    float tmax = -INFINITY;
    if (vmask == 0xFFFFFFFFu) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            sacc[e] *= ks[e];
            tmax = fmaxf(tmax, sacc[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
            sacc[e] = ((vmask >> key) & 1u) ? sacc[e] * ks[e] : -INFINITY;
            tmax = fmaxf(tmax, sacc[e]);
        }
    }
    {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * zch;
    }
    if (__ballot(tmax > st.m_run + kWideSlack)) {
        const bool over = __ballot(st.m_run != -INFINITY && tmax > st.m_run + kWideSlack) != 0;
        if (tmax > st.m_run + kWideSlack) st.m_run = tmax;
        if (over) return true;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        sacc[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], zch, -m_use));
        psum += sacc[e];
    }
    st.l_run += psum;
    // value weights carry the key scale: P'[key, head] = p * k_scale[key]
    u32x4 pb[2];
#pragma unroll
    for (int step = 0; step < 2; ++step)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            pb[step][t] = pack_bf16x2(sacc[8 * step + 2 * t] * ks[8 * step + 2 * t],
                                      sacc[8 * step + 2 * t + 1] * ks[8 * step + 2 * t + 1]);
    // transpose-load roles: this lane supplies, for element j = (lane % 16) / 2 of
    // its 16-lane group, the row of key(j) and the column half (lane & 1)
    const int li = lane & 15, gh = (lane >> 4) & 1;
    const int jj = li >> 1;
    const int krow = (jj < 4 ? 4 * kb + jj : 8 + 4 * kb + (jj - 4));
    const char* vsrc = tb + krow * C::PITCH + 16 * gh + 8 * (li & 1);
    typedef int v2i __attribute__((ext_vector_type(2)));
    constexpr int NPV = 2 * C::VT;
    constexpr int DVW = C::V_AHEAD;
    auto ldv = [&](int n) {
        const int step = n / C::VT, v = n % C::VT;
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(vsrc + 16 * step * C::PITCH + 32 * v));
    };
    v2i vw[DVW];
#pragma unroll
    for (int j = 0; j < DVW; ++j) vw[j] = ldv(j);
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
        const v2i raw = vw[n % DVW];
        if (n + DVW < NPV) vw[n % DVW] = ldv(n + DVW);
        const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[0], 1.f, false);
        const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[0], 1.f, true);
        const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[1], 1.f, false);
        const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[1], 1.f, true);
        const u32x4 va = {__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                          __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
        st.o[n % C::VT] = mfma32_bf16(va, pb[n / C::VT], st.o[n % C::VT]);
        __builtin_amdgcn_sched_barrier(0);
    }
    return false;
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void mla_fp8w_kernel(MlaArgs a)
{
    using C = Fp8WideCfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) u32x4 tiles[C::NBUF * C::BUF_CH];
    __shared__ uint32_t lrow[kMaxListLen];
    __shared__ uint32_t tmask[kMaxListLen / kTileKeys];
    __shared__ __attribute__((aligned(16))) float kscols[C::NW][kTileKeys];
    __shared__ int restart_flags[2];
    volatile int* restart = restart_flags;

    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int n_units = a.B * a.t_count * a.n_split * HB;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int hb = unit % HB;
    const int split = (unit / HB) % a.n_split;
    const int rq = unit / HB / a.n_split;
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;
    const int L = min(a.kv_len[b], a.Lmax);

    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    if (tid < 2) restart[tid] = 0;
    const int col = lane & 31, kb = lane >> 5;
    const int head = hb * kHeadsPerBlock + w * 32 + col;
    const bool head_ok = head < a.H;

    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);
    const int n_tiles = (j_end > j_begin && L > 0) ? (j_end - j_begin + kTileKeys - 1) / kTileKeys : 0;

    const char* kvb = (const char*)a.kv + (size_t)b * a.Lmax * C::ROWB;
    const int32_t* idxr = a.idx + row * a.K;
    constexpr int kListPer = kMaxListLen / C::NT;
    const int n_list = n_tiles * kTileKeys;
    const int j_last = max(j_end - 1, 0);
    int raw[kListPer];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) raw[r] = idxr[min(j_begin + tid + C::NT * r, j_last)];
    // Q^T operand: lane (col, kb) holds the codes of dims [64 s + 32 kb, + 32) of head `col`
    const size_t qrow = row * a.H + (head_ok ? head : 0);
    i32x8 qb[C::QS];
    {
        const char* src = (const char*)a.q + qrow * DQK + 32 * kb;
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
            const u32x4 lo = ld16(src + 64 * s), hi = ld16(src + 64 * s + 16);
            qb[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }
    const float zch = a.sm_scale * kLog2e * a.q_scale[qrow];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
        const int j = tid + C::NT * r;
        const int s = raw[r];
        const bool ok = j < n_list && j_begin + j < j_end && s >= 0 && s < L;
        lrow[j] = ok ? (uint32_t)s * C::ROWB : 0u;
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {
            tmask[j / kTileKeys] = (uint32_t)bits;
            tmask[j / kTileKeys + 1] = (uint32_t)(bits >> 32);
        }
    }
#pragma unroll
    for (int s = 0; s < C::QS; ++s) asm volatile("" : "+v"(qb[s]));
    barrier_lds();

    WideState<DQK, DV> st;
#pragma unroll
    for (int v = 0; v < C::VT; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    constexpr int AHEAD = C::NBUF - 1;

#pragma unroll 1
    for (;;) {
#pragma unroll
        for (int g = 0; g < AHEAD; ++g)
            if (g < n_tiles) gather_tile_asm<C>(kvb, lrow, g * kTileKeys, w, lane, tiles + g * C::BUF_CH);
        int cur = 0;
#pragma unroll 1
        for (int it = 0; it < n_tiles; ++it) {
            // tile `it` has landed everywhere (the gathers of the next min(AHEAD - 1,
            // n_tiles - 1 - it) tiles may still be in flight) and every wave is done
            // with the buffer computed in the previous iteration, refilled below
            const int later = min(AHEAD - 1, n_tiles - 1 - it);
            if (later >= 2)
                barrier_vm<2 * C::DMA>();
            else if (later == 1)
                barrier_vm<C::DMA>();
            else
                barrier_vm<0>();
            if (it > 0 && restart[(it - 1) & 1]) break;
            const uint32_t vm = tmask[it];
            const int nxt = cur == 0 ? C::NBUF - 1 : cur - 1;  // (cur + AHEAD) % NBUF
            PendingGather<C> pg;
            pg.kvb = kvb;
            pg.dst = tiles + nxt * C::BUF_CH;
            pg.lrow = lrow + min(it + AHEAD, n_tiles - 1) * kTileKeys;
            pg.active = it + AHEAD < n_tiles;
            pg.start(w, lane);
            if (tile_compute_fp8w<DQK, DV>(tiles + cur * C::BUF_CH, vm, qb, st, zch, lane, w, kscols[w], pg) &&
                lane == 0)
                restart[it & 1] = 1;
            cur = cur == C::NBUF - 1 ? 0 : cur + 1;
        }
        barrier_vm<0>();
        if (!(restart[0] | restart[1])) break;
        barrier_lds();
        if (tid < 2) restart[tid] = 0;
#pragma unroll
        for (int v = 0; v < C::VT; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
        st.l_run = 0.f;
    }
    mla_write_rows_wide<DQK, DV, C>(a, st, row, rq, split, head, head_ok, kb);
}

// ================================================================ fp8 kernel
// The bf16 kernel's structure on e4m3 operands: the latent cache rows and the
// queries as codes with one fp32 scale per row.  A cache row is DQK codes and
// then 16 bytes holding its scale, so the gather brings the scale with the row.
//   - QK^T runs on the 32x32x64 f8f6f4 MFMA (twice the bf16 rate): wave half 0
//     takes dims [0, D0), half 1 [D0, DQK), in 64-deep steps; both operands hold
//     32 consecutive dims per lane, so the contraction order inside a step is
//     the same for both.  Logit = S * k_scale[key] * q_scale[head] * sm_scale.
//   - PV stays on bf16 MFMA (e4m3 weights would cost up to 6% per weight).  The
//     8-bit transpose load gives a lane 8 keys of one value column (inside a
//     16-lane group, lane i receives byte j from the address of lane 2j + i/8,
//     at offset i%8), which convert exactly to bf16; the weights carry the key
//     scale, P'[key, head] = p * k_scale[key].
template <int DQK, int DV>
struct Fp8Cfg {
    static constexpr int ROWB = DQK + 16;       // bytes of a cache row (codes + scale)
    static constexpr int CPR = ROWB / 16;       // 16-byte chunks per row, scale chunk included
    static constexpr int PCH = CPR;             // LDS pitch in chunks (odd: conflict-free 16-byte columns)
    static constexpr int PITCH = PCH * 16;
    static constexpr int TILE_CH = kTileKeys * PCH;
    static constexpr int DMA_PER_WAVE = (TILE_CH + 511) / 512;
    static constexpr int STAGE_CH = kTileKeys * (DV * 2 + 16) / 16;  // the epilogue's 32 staged rows
    static constexpr int BUF_CH = DMA_PER_WAVE * 512 > STAGE_CH ? DMA_PER_WAVE * 512 : STAGE_CH;
    static constexpr int D0 = ((DQK / 64 + 1) / 2) * 64;        // dims of wave half 0
    static constexpr int NS0 = D0 / 64, NS1 = (DQK - D0) / 64;  // 64-deep steps of each half
    static constexpr int VH = DV / 2;
    static constexpr int VT = VH / 32;
    static_assert(DQK % 64 == 0 && DV % 64 == 0 && DV <= DQK && CPR % 2 == 1, "shape");
};

__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, f32x16 c)
{
    // formats 0/0: both operands OCP e4m3; unit block scales (127 = 2^0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int DQK, int DV>
__device__ __forceinline__ void tile_compute8(const u32x4* tile, uint32_t vmask,
                                              const i32x8 (&qb)[Fp8Cfg<DQK, DV>::NS0], float zch,
                                              Bf16State<DQK, DV>& st, float (*xbuf)[16][64], int w, int lane)
{
    using C = Fp8Cfg<DQK, DV>;
    asm volatile("" : "+v"(lane));  // lane-derived addresses are recomputed per tile, not kept live
    const int col = lane & 31, kb = lane >> 5, half = w & 1;
    const char* tb = reinterpret_cast<const char*>(tile);
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
    const char* kr = tb + col * C::PITCH + (half ? C::D0 : 0) + 32 * kb;
    const int ns = half ? C::NS1 : C::NS0;
#pragma unroll
    for (int s = 0; s < C::NS0; ++s) {
        if (s < ns) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + 64 * s);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + 64 * s + 16);
            const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            sacc = mfma32_fp8(a, qb[s], sacc);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) xbuf[w][e][lane] = sacc[e];
    barrier_lds();
    // lane holds keys 8*i + 4*kb + j (register 4*i + j) of head `col`; the key
    // scales sit after each row's codes in the tile
    float ks[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
        ks[e] = *reinterpret_cast<const float*>(tb + (8 * (e >> 2) + 4 * kb + (e & 3)) * C::PITCH + DQK);
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * kb + (e & 3);
        const float sv = (sacc[e] + xbuf[w ^ 1][e][lane]) * ks[e];
        sacc[e] = ((vmask >> key) & 1u) ? sv : -INFINITY;
        tmax = fmaxf(tmax, sacc[e]);
    }
    {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * zch;
    }
    if (__ballot(tmax > st.m_run + 8.f)) {
        const float m_new = fmaxf(st.m_run, tmax);
        const float alpha = st.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int v = 0; v < C::VT; ++v) st.o[v] *= alpha;
        st.m_run = m_new;
    }
    const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        sacc[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], zch, -m_use));
        psum += sacc[e];
    }
    st.l_run += psum;
    // transpose-load roles: this lane supplies, for element j = (lane % 16) / 2 of
    // its 16-lane group, the row of key(j) and the column half (lane & 1)
    const int li = lane & 15, gh = (lane >> 4) & 1;
    const int jj = li >> 1;
    const int krow = (jj < 4 ? 4 * kb + jj : 8 + 4 * kb + (jj - 4));
    const char* vsrc = tb + krow * C::PITCH + C::VH * half + 16 * gh + 8 * (li & 1);
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        u32x4 pb;
#pragma unroll
        for (int t = 0; t < 4; ++t)
            pb[t] = pack_bf16x2(sacc[8 * step + 2 * t] * ks[8 * step + 2 * t],
                                sacc[8 * step + 2 * t + 1] * ks[8 * step + 2 * t + 1]);
#pragma unroll
        for (int v = 0; v < C::VT; ++v) {
            typedef int v2i __attribute__((ext_vector_type(2)));
            const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(vsrc + 16 * step * C::PITCH + 32 * v));
            const f32x2 a01 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], false);
            const f32x2 a23 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], true);
            const f32x2 a45 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], false);
            const f32x2 a67 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], true);
            const u32x4 va = {pack_bf16x2(a01[0], a01[1]), pack_bf16x2(a23[0], a23[1]),
                              pack_bf16x2(a45[0], a45[1]), pack_bf16x2(a67[0], a67[1])};
            st.o[v] = mfma32_bf16(va, pb, st.o[v]);
        }
    }
}

// Same work unit, waves, list set-up, gather pipeline and epilogue as the bf16 kernel.
template <int DQK, int DV>
__global__ __launch_bounds__(512) void mla_fp8_kernel(MlaArgs a)
{
    using C = Fp8Cfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) u32x4 tA[C::BUF_CH];
    __shared__ __attribute__((aligned(16))) u32x4 tB[C::BUF_CH];
    __shared__ float xbuf[8][16][64];
    __shared__ uint32_t lrow[kMaxListLen];
    __shared__ uint32_t tmask[kMaxListLen / kTileKeys];

    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int n_units = a.B * a.t_count * a.n_split * HB;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int hb = unit % HB;
    const int split = (unit / HB) % a.n_split;
    const int rq = unit / HB / a.n_split;
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;
    const int L = min(a.kv_len[b], a.Lmax);

    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int pair = w >> 1, half = w & 1;
    const int col = lane & 31, kb = lane >> 5;
    const int head = hb * kHeadsPerBlock + pair * 32 + col;
    const bool head_ok = head < a.H;

    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);
    // an empty sequence (L = 0) has no row to gather, not even the stand-in row 0
    const int n_tiles = (j_end > j_begin && L > 0) ? (j_end - j_begin + kTileKeys - 1) / kTileKeys : 0;

    const char* kvb = (const char*)a.kv + (size_t)b * a.Lmax * C::ROWB;
    const int32_t* idxr = a.idx + row * a.K;
    constexpr int kListPer = kMaxListLen / 512;
    const int n_list = n_tiles * kTileKeys;
    const int j_last = max(j_end - 1, 0);
    int raw[kListPer];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) raw[r] = idxr[min(j_begin + tid + 512 * r, j_last)];
    // Q^T operand: head `head`, dims [D0 * half + 64 s + 32 kb, + 32) of step s
    // (half 1 reloads its last step for the unused fifth, so every load is valid)
    const size_t qrow = row * a.H + (head_ok ? head : 0);
    i32x8 qb[C::NS0];
    {
        const char* src = (const char*)a.q + qrow * DQK + (half ? C::D0 : 0) + 32 * kb;
        const int ns = half ? C::NS1 : C::NS0;
#pragma unroll
        for (int s = 0; s < C::NS0; ++s) {
            const char* p = src + 64 * min(s, ns - 1);
            const u32x4 lo = ld16(p), hi = ld16(p + 16);
            qb[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }
    const float zch = a.sm_scale * kLog2e * a.q_scale[qrow];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
        const int j = tid + 512 * r;
        const int s = raw[r];
        const bool ok = j < n_list && j_begin + j < j_end && s >= 0 && s < L;
        lrow[j] = ok ? (uint32_t)s * C::ROWB : 0u;
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {  // j is a multiple of 64 here, so both words lie inside tmask
            tmask[j / kTileKeys] = (uint32_t)bits;
            tmask[j / kTileKeys + 1] = (uint32_t)(bits >> 32);
        }
    }
    barrier_lds();

    Bf16State<DQK, DV> st;
#pragma unroll
    for (int v = 0; v < C::VT; ++v)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    if (n_tiles > 0) gather_tile<C>(kvb, lrow, 0, w, lane, tA);
#pragma unroll 1
    for (int it = 0; it < n_tiles; it += 2) {
        barrier_lds_vm();
        const uint32_t vmA = tmask[it];
        if (it + 1 < n_tiles) gather_tile<C>(kvb, lrow, (it + 1) * kTileKeys, w, lane, tB);
        __builtin_amdgcn_sched_barrier(0);
        tile_compute8<DQK, DV>(tA, vmA, qb, zch, st, xbuf, w, lane);
        if (it + 1 >= n_tiles) break;
        barrier_lds_vm();
        const uint32_t vmB = tmask[it + 1];
        if (it + 2 < n_tiles) gather_tile<C>(kvb, lrow, (it + 2) * kTileKeys, w, lane, tA);
        __builtin_amdgcn_sched_barrier(0);
        tile_compute8<DQK, DV>(tB, vmB, qb, zch, st, xbuf, w, lane);
    }
    mla_write_rows<DQK, DV, C>(a, st, tA, tB, hb, row, rq, split, head, head_ok, pair, half, col, kb, tid);
}

// ================================================================ fp32 kernel
template <int DQK, int DV>
struct F32Cfg {
    static constexpr int ROWB = DQK * 4;
    static constexpr int CPR = ROWB / 16;
    static constexpr int PITCH = ROWB + 16;
    static constexpr int SHB = ROWB / 4;
    static constexpr int QCH = SHB / 16;
    static constexpr int VT = DV / 16;
    static_assert(ROWB % 64 == 0 && DV % 16 == 0 && DV <= DQK, "shape");
};

template <int DQK, int DV>
__global__ __launch_bounds__(64) void mla_f32_kernel(MlaArgs a)
{
    using C = F32Cfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) char tile[kTileKeys * C::PITCH];
    __shared__ int sidx[kTileKeys];

    const int HG = (a.H + 15) / 16;
    const int n_units = a.B * a.t_count * a.n_split * HG;
    const int unit = xcd_unit(blockIdx.x, n_units);
    if (unit >= n_units) return;
    const int hg = unit % HG;
    const int split = (unit / HG) % a.n_split;
    const int rq = unit / HG / a.n_split;
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;
    const int L = min(a.kv_len[b], a.Lmax);
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int head = hg * 16 + n;
    const bool head_ok = head < a.H;
    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);

    u32x4 qb[C::QCH];
    {
        const char* src = (const char*)a.q + ((row * a.H + (head_ok ? head : 0)) * DQK) * 4 + g * C::SHB;
#pragma unroll
        for (int c = 0; c < C::QCH; ++c) qb[c] = head_ok ? ld16(src + 16 * c) : u32x4{0, 0, 0, 0};
    }
    f32x4 o[C::VT];
#pragma unroll
    for (int v = 0; v < C::VT; ++v) o[v] = f32x4{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.f;
    const float zc = a.sm_scale * kLog2e;
    const char* kvb = (const char*)a.kv + (size_t)b * a.Lmax * C::ROWB;
    const int32_t* idxr = a.idx + row * a.K;

#pragma unroll 1
    for (int j0 = j_begin; j0 < j_end; j0 += kTileKeys) {
        if (lane < kTileKeys) sidx[lane] = valid_key(a, idxr, j0 + lane, j_end, L);
        __syncthreads();
        for (int c = lane; c < kTileKeys * C::CPR; c += 64) {
            const int r = c / C::CPR, cc = c % C::CPR;
            const int s = sidx[r];
            const u32x4 v = s >= 0 ? ld16(kvb + (size_t)s * C::ROWB + cc * 16) : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(&tile[r * C::PITCH + cc * 16]) = v;
        }
        __syncthreads();
        f32x4 s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x4 acc = f32x4{0, 0, 0, 0};
            const char* kr = &tile[(16 * mt + n) * C::PITCH + g * C::SHB];
#pragma unroll
            for (int c = 0; c < C::QCH; ++c) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(kr + 16 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(ka[e]), __uint_as_float(qb[c][e]), acc);
            }
            s[mt] = acc;
        }
        float z[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[mt][i] = sidx[16 * mt + 4 * g + i] >= 0 ? s[mt][i] * zc : -INFINITY;
                tmax = fmaxf(tmax, z[mt][i]);
            }
        tmax = group4_max(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[mt][i] = exp2f(z[mt][i] - m_use);
                psum += z[mt][i];
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int v = 0; v < C::VT; ++v) o[v] *= alpha;
        // O^T += V^T . P^T in eight 4-key steps; step st pairs lane group g with key
        // 4g + st (st < 4) or 16 + 4g + st - 4, the keys whose logits the lane holds
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const int key = st < 4 ? 4 * g + st : 16 + 4 * g + (st - 4);
            const float pv = st < 4 ? z[0][st] : z[1][st - 4];
            const float* vr = reinterpret_cast<const float*>(&tile[key * C::PITCH]);
#pragma unroll
            for (int v = 0; v < C::VT; ++v) o[v] = mfma_f32(vr[16 * v + n], pv, o[v]);
        }
        __syncthreads();
    }

    const float l_tot = group4_sum(l_run);
    if (!head_ok) return;
    const size_t orow = row * a.H + head;
    if (a.n_split == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int v = 0; v < C::VT; ++v)
            *reinterpret_cast<f32x4*>((float*)a.out + orow * DV + 16 * v + 4 * g) = o[v] * inv;
        if (a.lse && g == 0) a.lse[orow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
        using P = PartRow<kF32, DV>;
        float* pr = (float*)((char*)a.part + (((size_t)rq * a.n_split + split) * a.H + head) * P::bytes);
#pragma unroll
        for (int v = 0; v < C::VT; ++v) *reinterpret_cast<f32x4*>(pr + 16 * v + 4 * g) = o[v];
        if (g == 0) {
            pr[DV] = m_run;
            pr[DV + 1] = l_tot;
        }
    }
}

// ============================================================ split combine
// One wave per (query, head): merge the split partials by log-sum-exp.  Lane sp
// holds the weight of split sp (for bf16 rows, whose values are already divided by
// their own sum, the weight carries that sum).  Each lane owns 16-byte chunks of
// the value row; the chunks of up to four splits are loaded before any is used,
// the first batch together with the (m, l) pairs.  Partials are read once and
// outputs written once: both carry the non-temporal hint (measured on bf16
// outputs: decode at 32K context, step 181.3 -> 180.4 us; at 128K 120.2 -> 119.9 us).
template <int DT, int DV>
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a)
{
    using P = PartRow<DT, DV>;
    constexpr int EPC = DT == kBF16 ? 8 : 4;  // values per 16-byte chunk
    constexpr int NCK = P::vbytes / 16;       // chunks per value row
    constexpr int CPL = (NCK + 63) / 64;      // chunks per lane
    constexpr int kBatch = 4;
    // blocks go to the XCDs in contiguous eighths, as the MLA units do, so a query's
    // partials are read on the XCD whose L2 received them
    const int wid = xcd_unit(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    const int lane = lane_id();
    if (wid >= a.B * a.t_count * a.H) return;
    const int head = wid % a.H, rq = wid / a.H;
    const int b = rq / a.t_count, t = a.t_begin + rq % a.t_count;
    const size_t orow = ((size_t)b * a.T + t) * a.H + head;
    const char* base = (const char*)a.part + ((size_t)rq * a.n_split * a.H + head) * P::bytes;
    const size_t sstride = (size_t)a.H * P::bytes;
    const int ns = a.n_split;

    const float* ml = (const float*)(base + (size_t)(lane < ns ? lane : 0) * sstride + P::vbytes);
    const float mi0 = ml[0], li0 = ml[1];
    u32x4 v[kBatch][CPL];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const char* rowp = base + (size_t)min(s0 + j, ns - 1) * sstride;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                v[j][k] = (NCK % 64 == 0 || c < NCK) ? ld16_nt(rowp + 16 * c) : u32x4{0, 0, 0, 0};
            }
        }
    };
    load_batch(0);
    __builtin_amdgcn_sched_barrier(0);  // keep the value loads ahead of the weight reductions

    const float mi = lane < ns ? mi0 : -INFINITY;
    const float li = lane < ns ? li0 : 0.f;
    const float M = wave_max(mi);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float ei = lane < ns ? exp2f(mi - Mu) : 0.f;
    const float Ls = wave_sum(ei * li);
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    const float wi = (DT == kBF16 ? ei * li : ei) * inv;  // weight of a stored value row

    float acc[CPL][EPC];
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[k][e] = 0.f;
    for (int s0 = 0;;) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            // split s0 + j's weight (zero past the last split) from its lane
            const float wsp = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wi), min(s0 + j, 63)));
            const float wj = s0 + j < ns ? wsp : 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = v[j][k][e];
                    if constexpr (DT == kBF16) {
                        acc[k][2 * e] = fmaf(wj, __uint_as_float(x << 16), acc[k][2 * e]);
                        acc[k][2 * e + 1] = fmaf(wj, __uint_as_float(x & 0xFFFF0000u), acc[k][2 * e + 1]);
                    } else {
                        acc[k][e] = fmaf(wj, __uint_as_float(x), acc[k][e]);
                    }
                }
        }
        s0 += kBatch;
        if (s0 >= ns) break;
        load_batch(s0);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        if (NCK % 64 != 0 && c >= NCK) continue;
        if constexpr (DT == kBF16) {
            const u32x4 w4 = {pack_bf16x2(acc[k][0], acc[k][1]), pack_bf16x2(acc[k][2], acc[k][3]),
                              pack_bf16x2(acc[k][4], acc[k][5]), pack_bf16x2(acc[k][6], acc[k][7])};
            st16_nt((uint16_t*)a.out + orow * DV + 8 * c, w4);
        } else {
            st16_nt((float*)a.out + orow * DV + 4 * c, u32x4{__float_as_uint(acc[k][0]), __float_as_uint(acc[k][1]),
                                                          __float_as_uint(acc[k][2]), __float_as_uint(acc[k][3])});
        }
    }
    if (a.lse && lane == 0) a.lse[orow] = Ls > 0.f ? (Mu + log2f(Ls)) * kLn2 : -INFINITY;
}

template <int DT, int DV>
hipError_t launch_combine(const MlaArgs& a, hipStream_t s)
{
    if (a.n_split == 1) return hipSuccess;
    const long long waves = (long long)a.B * a.t_count * a.H;
    const long long blocks = (waves + 3) / 4;
    mla_combine_kernel<DT, DV><<<dim3((unsigned)(8 * ((blocks + 7) / 8))), 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_bf16(const MlaArgs& a, hipStream_t s)
{
    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const long long units = (long long)a.B * a.t_count * a.n_split * HB;
    mla_bf16_kernel<DQK, DV><<<dim3((unsigned)(8 * ((units + 7) / 8))), 512, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine<kBF16, DV>(a, s);
}

template <int DQK, int DV>
hipError_t launch_wide(const MlaArgs& a, hipStream_t s)
{
    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const long long units = (long long)a.B * a.t_count * a.n_split * HB;
    // one query per sequence: every gathered row is read by one workgroup only, and
    // non-temporal gathers measured faster (decode at 32K context: step 183.4 ->
    // 179.0 us); prefill queries share rows through L2 (5.7% slower with the hint)
    const dim3 grid((unsigned)(8 * ((units + 7) / 8)));
    if (a.t_count == 1)
        mla_wide_kernel<DQK, DV, true><<<grid, 256, 0, s>>>(a);
    else
        mla_wide_kernel<DQK, DV, false><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine<kBF16, DV>(a, s);
}

// Tiles of one split's index list.  The wide kernels win on long lists; on the
// 4-tile lists of a 16-way split (16 decode queries at K = 2048) the bf16 wide
// kernel measured 31.1 us against 29.4-29.8 us for the two-waves-per-SIMD one.
int split_tiles(const MlaArgs& a)
{
    const int per = (a.K + a.n_split - 1) / a.n_split;
    return (per + kTileKeys - 1) / kTileKeys;
}
constexpr int kWideMinTiles = 8;

template <int DQK, int DV>
hipError_t launch_fp8(const MlaArgs& a, hipStream_t s)
{
    const int HB = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const long long units = (long long)a.B * a.t_count * a.n_split * HB;
    const dim3 grid((unsigned)(8 * ((units + 7) / 8)));
    if (split_tiles(a) >= kWideMinTiles)
        mla_fp8w_kernel<DQK, DV><<<grid, 256, 0, s>>>(a);
    else
        mla_fp8_kernel<DQK, DV><<<grid, 512, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine<kBF16, DV>(a, s);
}

template <int DQK, int DV>
hipError_t launch_f32(const MlaArgs& a, hipStream_t s)
{
    const int HG = (a.H + 15) / 16;
    const long long units = (long long)a.B * a.t_count * a.n_split * HG;
    mla_f32_kernel<DQK, DV><<<dim3((unsigned)(8 * ((units + 7) / 8))), 64, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine<kF32, DV>(a, s);
}

}  // namespace

bool mla_supported(int dtype, int Dqk, int Dv)
{
    if (dtype == kF32) return Dqk == 80 && Dv == 64;
    if (dtype == kBF16) return (Dqk == 576 && Dv == 512) || (Dqk == 192 && Dv == 128);
    if (dtype == kFP8) return Dqk == 576 && Dv == 512;
    return false;
}

// Split the index list only when the queries alone leave CUs idle.
int mla_split_count(int B, int t_count, int H, int K)
{
    const long long hb = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const long long units = (long long)B * t_count * hb;
    long long ns = (256 + units - 1) / units;
    const long long max_ns = K / 128 > 1 ? K / 128 : 1;
    if (ns > max_ns) ns = max_ns;
    if (ns > 16) ns = 16;
    return (int)(ns < 1 ? 1 : ns);
}

size_t mla_partial_bytes(int dtype, int B, int t_count, int H, int Dv, int n_split)
{
    if (n_split <= 1) return 0;
    return (size_t)B * t_count * n_split * H * ((size_t)Dv * (dtype == kF32 ? 4 : 2) + 16);
}

hipError_t launch_mla(int dtype, const MlaArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    if (dtype == kF32) return launch_f32<80, 64>(a, s);
    if (dtype == kFP8) return launch_fp8<576, 512>(a, s);
    if (a.Dqk == 192) return launch_bf16<192, 128>(a, s);
    if (split_tiles(a) >= kWideMinTiles) return launch_wide<576, 512>(a, s);
    return launch_bf16<576, 512>(a, s);
}

}  // namespace dsa
