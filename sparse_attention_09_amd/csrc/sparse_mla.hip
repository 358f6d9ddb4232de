// sparse_mla.hip -- sparse absorbed-latent MLA forward on gfx950 MFMA.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 2:
// main MLA attention runs only over each query's selected tokens, which with a
// sparse kernel costs O(index_topk) per query instead of O(L).  Absorbed form:
// one latent row kv[s] = [c_kv (Dv) | k_rope] is the key of every head and its
// first Dv columns are the value, so all heads of a query share each gathered
// row:  z_j = sm_scale * q_h . kv[idx_j],  o_h = sum_j softmax(z)_j kv[idx_j, :Dv].
//
// Work item = (query, group of 16*NW heads, split of the index list).  Per
// 32-entry tile: the selected rows are gathered (coalesced 16-byte loads of
// whole rows) into an LDS tile; each wave (16 heads) computes
//   S^T[32 keys x 16 heads] = K_tile . Q^T        (keys on M, heads on N)
// so a lane holds one head's logits for 8 keys, runs the online softmax in
// registers, and feeds P^T directly as the B operand of
//   O^T[Dv x 16 heads] += V^T . P^T               (value dims on M)
// whose A operand (V^T) is read from the row-major tile with the LDS transpose
// load; the key order inside the contraction is permuted to match the lanes'
// logits.  Queries' heads of one (query, split) unit are launched on the same
// XCD so the second head group finds the gathered rows in that XCD's L2.
// Splits write fp32 partials (unnormalised O, running max, running sum) that a
// combine kernel merges by log-sum-exp.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTileKeys = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT> struct MlaElem;
template <> struct MlaElem<kF32> { static constexpr int v = 4; };
template <> struct MlaElem<kBF16> { static constexpr int v = 2; };

template <int DT, int DQK, int DV, int NW>
struct MlaCfg {
    static constexpr int EB = MlaElem<DT>::v;
    static constexpr int ROWB = DQK * EB;        // bytes of one latent row
    static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
    static constexpr int PITCH = ROWB + 16;      // padded LDS row pitch
    static constexpr int SHB = ROWB / 4;         // bytes of a lane's contraction share
    static constexpr int QCH = SHB / 16;         // 16-byte chunks in that share
    static constexpr int VT = DV / 16;           // value-dim tiles of 16
    static constexpr int NT = NW * 64;           // threads
    static constexpr int HPB = 16 * NW;          // heads per block
    static_assert(ROWB % 64 == 0, "row share must be whole 16-byte chunks");
    static_assert(DV % 16 == 0 && DV <= DQK, "value width");
};

// Work-item decode with XCD grouping: blocks L, L+8, ... land on one XCD, so
// all head groups of a (query, split) unit share L2.
__device__ __forceinline__ void mla_item(int L, int HG, int& unit, int& hg)
{
    const int xcd = L & 7, rest = L >> 3;
    hg = rest % HG;
    unit = (rest / HG) * 8 + xcd;
}

template <int DT, int DQK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void mla_kernel(MlaArgs a)
{
    using C = MlaCfg<DT, DQK, DV, NW>;
    __shared__ __attribute__((aligned(16))) char tile[kTileKeys * C::PITCH];
    __shared__ int sidx[kTileKeys];

    const int HG = (a.H + C::HPB - 1) / C::HPB;
    int unit, hg;
    mla_item(blockIdx.x, HG, unit, hg);
    const int n_units = a.B * a.t_count * a.n_split;
    if (unit >= n_units) return;
    const int split = unit % a.n_split;
    const int rq = unit / a.n_split;            // query row within this launch
    const int b = rq / a.t_count;
    const int t = a.t_begin + rq % a.t_count;
    const size_t row = (size_t)b * a.T + t;     // row of the full [B,T,...] tensors
    const int L = min(a.kv_len[b], a.Lmax);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int head = hg * C::HPB + wave * 16 + n;
    const bool head_ok = head < a.H;

    // split range over the index list, whole tiles
    const int per = ((a.K + a.n_split - 1) / a.n_split + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int j_begin = split * per;
    const int j_end = min(a.K, j_begin + per);

    // Q^T operand: lane holds head `head`, contraction share g.
    u32x4 qb[C::QCH];
    {
        const char* src = (const char*)a.q + ((row * a.H + (head_ok ? head : 0)) * DQK) * C::EB + g * C::SHB;
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
        if (tid < kTileKeys) {
            const int j = j0 + tid;
            int s = j < j_end ? idxr[j] : -1;
            sidx[tid] = (s >= 0 && s < L) ? s : -1;
        }
        __syncthreads();
        // gather the tile's rows (invalid rows become zeros)
        for (int c = tid; c < kTileKeys * C::CPR; c += C::NT) {
            const int r = c / C::CPR, col = c % C::CPR;
            const int s = sidx[r];
            const u32x4 v = s >= 0 ? ld16(kvb + (size_t)s * C::ROWB + col * 16) : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(&tile[r * C::PITCH + col * 16]) = v;
        }
        __syncthreads();

        // S^T = K_tile . Q^T for two 16-key M tiles
        f32x4 s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x4 acc = f32x4{0, 0, 0, 0};
            const char* kr = &tile[(16 * mt + n) * C::PITCH + g * C::SHB];
#pragma unroll
            for (int c = 0; c < C::QCH; ++c) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(kr + 16 * c);
                if constexpr (DT == kBF16) {
                    acc = mfma_bf16(ka, qb[c], acc);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(ka[e]), __uint_as_float(qb[c][e]), acc);
                }
            }
            s[mt] = acc;
        }

        // online softmax (log2 domain); lane holds keys 16*mt + 4*g + i of head `head`
        float z[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = sidx[16 * mt + 4 * g + i] >= 0;
                z[mt][i] = ok ? s[mt][i] * zc : -INFINITY;
                tmax = fmaxf(tmax, z[mt][i]);
            }
        tmax = group4_max(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[mt][i] = exp2f(z[mt][i] - m_use);
                psum += p[mt][i];
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int v = 0; v < C::VT; ++v) o[v] *= alpha;
        }

        // O^T += V^T . P^T
        if constexpr (DT == kBF16) {
            u32x4 pb;
            pb[0] = pack_bf16x2(p[0][0], p[0][1]);
            pb[1] = pack_bf16x2(p[0][2], p[0][3]);
            pb[2] = pack_bf16x2(p[1][0], p[1][1]);
            pb[3] = pack_bf16x2(p[1][2], p[1][3]);
            // transpose-load addresses: this lane supplies row key_j = 4g + j (and 16 + 4g + j),
            // columns 16*vt + 4q, for j = n / 4, q = n % 4
            const int jr = n >> 2, qc = n & 3;
            const char* r1 = &tile[(4 * g + jr) * C::PITCH + 8 * qc];
            const char* r2 = &tile[(16 + 4 * g + jr) * C::PITCH + 8 * qc];
#pragma unroll
            for (int v = 0; v < C::VT; ++v) {
                const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(r1 + 32 * v));
                const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(r2 + 32 * v));
                const u32x2 y1 = __builtin_bit_cast(u32x2, x1);
                const u32x2 y2 = __builtin_bit_cast(u32x2, x2);
                o[v] = mfma_bf16(u32x4{y1[0], y1[1], y2[0], y2[1]}, pb, o[v]);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const int key = st < 4 ? 4 * g + st : 16 + 4 * g + (st - 4);
                const float pv = st < 4 ? p[0][st] : p[1][st - 4];
                const float* vr = reinterpret_cast<const float*>(&tile[key * C::PITCH]);
#pragma unroll
                for (int v = 0; v < C::VT; ++v) o[v] = mfma_f32(vr[16 * v + n], pv, o[v]);
            }
        }
        __syncthreads();
    }

    const float l_tot = group4_sum(l_run);
    if (!head_ok) return;
    const size_t orow = row * a.H + head;
    if (a.n_split == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int v = 0; v < C::VT; ++v) {
            const int d0 = 16 * v + 4 * g;
            if constexpr (DT == kBF16) {
                u32x2 w2 = {pack_bf16x2(o[v][0] * inv, o[v][1] * inv), pack_bf16x2(o[v][2] * inv, o[v][3] * inv)};
                *reinterpret_cast<u32x2*>((char*)a.out + (orow * DV + d0) * 2) = w2;
            } else {
                *reinterpret_cast<f32x4*>((float*)a.out + orow * DV + d0) = o[v] * inv;
            }
        }
        if (a.lse && g == 0) a.lse[orow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
        // partial record: O[DV] (unnormalised), m (log2 domain), l
        float* pr = a.part + (((size_t)rq * a.n_split + split) * a.H + head) * (DV + 2);
#pragma unroll
        for (int v = 0; v < C::VT; ++v) *reinterpret_cast<f32x4*>(pr + 16 * v + 4 * g) = o[v];
        if (g == 0) {
            pr[DV] = m_run;
            pr[DV + 1] = l_tot;
        }
    }
}

// Merge split partials: one wave per (query, head).
template <int DT, int DV>
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a)
{
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = lane_id();
    if (wid >= a.B * a.t_count * a.H) return;
    const int head = wid % a.H, rq = wid / a.H;
    const int b = rq / a.t_count, t = a.t_begin + rq % a.t_count;
    const size_t orow = ((size_t)b * a.T + t) * a.H + head;
    const float* base = a.part + ((size_t)rq * a.n_split * a.H + head) * (DV + 2);
    const size_t sstride = (size_t)a.H * (DV + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, base[sp * sstride + DV]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f;
    for (int sp = 0; sp < a.n_split; ++sp) Ls += exp2f(base[sp * sstride + DV] - Mu) * base[sp * sstride + DV + 1];
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    for (int d = lane; d < DV; d += 64) {
        float acc = 0.f;
        for (int sp = 0; sp < a.n_split; ++sp) acc += exp2f(base[sp * sstride + DV] - Mu) * base[sp * sstride + d];
        acc *= inv;
        if constexpr (DT == kBF16)
            ((uint16_t*)a.out)[orow * DV + d] = f32_to_bf16(acc);
        else
            ((float*)a.out)[orow * DV + d] = acc;
    }
    if (a.lse && lane == 0) a.lse[orow] = Ls > 0.f ? (Mu + log2f(Ls)) * kLn2 : -INFINITY;
}

template <int DT, int DQK, int DV, int NW>
hipError_t launch_cfg(const MlaArgs& a, hipStream_t s)
{
    using C = MlaCfg<DT, DQK, DV, NW>;
    const int HG = (a.H + C::HPB - 1) / C::HPB;
    const long long units = (long long)a.B * a.t_count * a.n_split;
    const long long blocks = 8LL * HG * ((units + 7) / 8);
    mla_kernel<DT, DQK, DV, NW><<<dim3((unsigned)blocks), C::NT, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    const long long waves = (long long)a.B * a.t_count * a.H;
    mla_combine_kernel<DT, DV><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool mla_supported(int dtype, int Dqk, int Dv)
{
    if (dtype == kF32) return Dqk == 80 && Dv == 64;
    if (dtype == kBF16) return (Dqk == 576 && Dv == 512) || (Dqk == 192 && Dv == 128);
    return false;
}

int mla_split_count(int B, int t_count, int H, int K)
{
    const long long hg = (H + 63) / 64;
    const long long units = (long long)B * t_count * hg;
    long long ns = (512 + units - 1) / units;
    const long long max_ns = K / 128 > 1 ? K / 128 : 1;
    if (ns > max_ns) ns = max_ns;
    if (ns > 16) ns = 16;
    return (int)(ns < 1 ? 1 : ns);
}

size_t mla_partial_bytes(int B, int t_count, int H, int Dv, int n_split)
{
    if (n_split <= 1) return 0;
    return (size_t)B * t_count * n_split * H * (Dv + 2) * sizeof(float);
}

hipError_t launch_mla(int dtype, const MlaArgs& a, hipStream_t s)
{
    if (a.t_count <= 0 || a.B <= 0) return hipSuccess;
    if (dtype == kF32) return launch_cfg<kF32, 80, 64, 1>(a, s);
    if (a.Dqk == 192) return launch_cfg<kBF16, 192, 128, 4>(a, s);
    return launch_cfg<kBF16, 576, 512, 4>(a, s);
}

}  // namespace dsa
