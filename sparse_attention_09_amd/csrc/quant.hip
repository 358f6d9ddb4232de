// quant.hip -- e4m3 quantisation: Hadamard-rotated indexer operands, and the
// unrotated MLA latent rows and queries of the fp8 attention.
//
// DeepSeek-V3.2 model documentation, "DeepSeek Sparse Attention (DSA)", item 1:
// the reference indexer runs in FP8 after an orthogonal Hadamard transform of
// q and k, so q.k is unchanged before quantisation.  Per row of length dim:
//   x' = fp32(H x),  H = Sylvester Hadamard / sqrt(dim)
//   amax = max|x'|;  amax == 0 -> codes 0, scale 1
//   else r = fp32(448 / amax), code_i = e4m3_rne_saturate(fp32(x'_i * r)),
//        scale = fp32(amax / 448).
// The same transform feeds the index-key cache update that precedes the indexer:
// a sequence's new key rows are quantised straight into their cache rows.
// The transform is the in-place butterfly, carried in fp64
// so that its only rounding before the final fp32 is the 1/sqrt(dim) scaling;
// the fp32 divisions are correctly rounded.  e4m3 (OCP E4M3FN: bias 7, max 448,
// no infinities) is encoded from the fp32 bit pattern with round-half-even.
#include "dsa_common.h"
#include "dsa_kernels.h"

#include <algorithm>

namespace dsa {
namespace {

__device__ __forceinline__ uint8_t e4m3_encode(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    const float a = fabsf(y);
    if (a >= 448.f) return sign | 0x7E;
    if (a < 0.015625f) {                       // below 2^-6: subnormal steps of 2^-9
        const float q = rintf(a * 512.f);       // exact scaling, ties to even
        return sign | (uint8_t)q;               // 8 -> 0x08, the smallest normal
    }
    const uint32_t ua = __float_as_uint(a);
    int e = (int)(ua >> 23) - 127;              // -6 .. 8
    const uint32_t mant = ua & 0x7FFFFFu;
    uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    if (q == 8u) {
        q = 0u;
        ++e;
    }
    return sign | (uint8_t)(((e + 7) << 3) | (int)q);
}

// Destination of input row `row`: the same row, or for a cache append (t_new > 0)
// cache row kv_len[b] - t_new + t of sequence b = row / t_new (t = row % t_new)
// in a [B, max_kv] cache; -1 when that row lies outside the cache.
struct RowMap {
    const int32_t* kv_len;
    int t_new, max_kv;
    __device__ __forceinline__ int64_t operator()(int64_t row) const
    {
        if (t_new <= 0) return row;
        const int64_t b = row / t_new;
        const int p = kv_len[b] - t_new + (int)(row - b * t_new);
        return (p >= 0 && p < max_kv) ? b * max_kv + p : -1;
    }
};

// Lane layout: each lane holds 8 consecutive elements of a row (element index
// i = 8 * li + j for lane li of the row's LPR = DIM / 8 lanes), a wave holds
// 64 / LPR rows.  The butterfly stages h = 1, 2, 4 pair elements inside a lane,
// the stages h >= 8 pair lanes li and li ^ (h / 8) of the same row.  Stages run
// in increasing h with the same pairing and signs whatever the layout, so every
// element goes through the same fp64 operations as in the plain transform.
// Blocks blk of nblk (of the launch's 256-thread blocks) share the rows.
template <int DIM, int XT>
__device__ __forceinline__ void rotate_quant_rows(int64_t rows, const void* x, uint8_t* codes, float* scales,
                                                  double inv_sqrt_dim, RowMap map, int blk, int nblk)
{
    constexpr int LPR = DIM / 8;   // lanes per row
    constexpr int RPW = 64 / LPR;  // rows per wave
    static_assert(DIM % 8 == 0 && LPR >= 1 && LPR <= 64, "dim");
    const int lane = lane_id(), li = lane % LPR, grp = lane / LPR;
    const int64_t wave = (int64_t)blk * 4 + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)nblk * 4;
    for (int64_t row0 = wave * RPW; row0 < rows; row0 += n_waves * RPW) {
        const int64_t row = row0 + grp;
        const int64_t orow = row < rows ? map(row) : -1;
        double v[8];
        if (orow >= 0) {
            if constexpr (XT == kBF16) {
                const u32x4 raw = ld16((const uint16_t*)x + row * DIM + 8 * li);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[2 * k] = (double)__uint_as_float(raw[k] << 16);
                    v[2 * k + 1] = (double)__uint_as_float(raw[k] & 0xFFFF0000u);
                }
            } else {
                const u32x4 r0 = ld16((const float*)x + row * DIM + 8 * li);
                const u32x4 r1 = ld16((const float*)x + row * DIM + 8 * li + 4);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[k] = (double)__uint_as_float(r0[k]);
                    v[4 + k] = (double)__uint_as_float(r1[k]);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = 0.0;
        }
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k & h) continue;
                const double a0 = v[k], b0 = v[k + h];
                v[k] = a0 + b0;
                v[k + h] = a0 - b0;
            }
#pragma unroll
        for (int hl = 1; hl < LPR; hl <<= 1)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const double o = __shfl_xor(v[k], hl, 64);
                v[k] = (li & hl) ? (o - v[k]) : (v[k] + o);
            }
        float xf[8];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            xf[k] = (float)(v[k] * inv_sqrt_dim);
            amax = fmaxf(amax, fabsf(xf[k]));
        }
#pragma unroll
        for (int hl = 1; hl < LPR; hl <<= 1) amax = fmaxf(amax, __shfl_xor(amax, hl, 64));
        if (orow >= 0) {
            const bool zero = amax == 0.f;
            const float r = zero ? 0.f : 448.f / amax;
            uint32_t packed[2] = {0u, 0u};
            if (!zero)
#pragma unroll
                for (int k = 0; k < 8; ++k) packed[k >> 2] |= (uint32_t)e4m3_encode(xf[k] * r) << (8 * (k & 3));
            *reinterpret_cast<u32x2*>(codes + orow * DIM + 8 * li) = u32x2{packed[0], packed[1]};
            if (li == 0) scales[orow] = zero ? 1.f : amax / 448.f;
        }
    }
}

// Optional words cleared by a launch beside its own work (a following top-k's
// counters): a grid-stride loop over the launch's threads.
struct ClearWords {
    uint32_t* p;
    long long n;
    __device__ __forceinline__ void run() const
    {
        if (p == nullptr) return;
        const long long nthreads = (long long)gridDim.x * blockDim.x;
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += nthreads) p[i] = 0u;
    }
};

template <int DIM, int XT>
__global__ __launch_bounds__(256) void rotate_quant_kernel(int64_t rows, const void* x, uint8_t* codes,
                                                           float* scales, double inv_sqrt_dim, RowMap map,
                                                           ClearWords clear)
{
    clear.run();
    rotate_quant_rows<DIM, XT>(rows, x, codes, scales, inv_sqrt_dim, map, blockIdx.x, gridDim.x);
}

// Per-row e4m3 quantisation without rotation (the codec above on the rows as
// they are).  One wave per row; lane li holds the 8-element chunks li and li + 64
// (rows of up to 1024 elements).  Codes go to codes + row * cpitch; the row scale
// to scales[row], or with `tail` into the 16 bytes after the row's codes (fp32
// scale, then 12 zero bytes: the fp8 latent-cache row layout).
template <int XT>
__device__ __forceinline__ void quant_rows_body(int64_t rows, int dim, const void* x, uint8_t* codes, int64_t cpitch,
                                                float* scales, int tail, int blk, int nblk)
{
    const int lane = lane_id(), nch = dim / 8;
    const int64_t n_waves = (int64_t)nblk * 4;
    for (int64_t row = (int64_t)blk * 4 + (threadIdx.x >> 6); row < rows; row += n_waves) {
        float xf[2][8];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = lane + 64 * k;
            if (c < nch) {
                if constexpr (XT == kBF16) {
                    const u32x4 raw = ld16((const uint16_t*)x + row * dim + 8 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xf[k][2 * e] = __uint_as_float(raw[e] << 16);
                        xf[k][2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
                    }
                } else {
                    const u32x4 r0 = ld16((const float*)x + row * dim + 8 * c);
                    const u32x4 r1 = ld16((const float*)x + row * dim + 8 * c + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xf[k][e] = __uint_as_float(r0[e]);
                        xf[k][4 + e] = __uint_as_float(r1[e]);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[k][e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xf[k][e]));
        }
        amax = wave_max(amax);
        const bool zero = amax == 0.f;
        const float r = zero ? 0.f : 448.f / amax;
        uint8_t* crow = codes + row * cpitch;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = lane + 64 * k;
            if (c >= nch) continue;
            uint32_t packed[2] = {0u, 0u};
            if (!zero)
#pragma unroll
                for (int e = 0; e < 8; ++e) packed[e >> 2] |= (uint32_t)e4m3_encode(xf[k][e] * r) << (8 * (e & 3));
            *reinterpret_cast<u32x2*>(crow + 8 * c) = u32x2{packed[0], packed[1]};
        }
        if (lane == 0) {
            const float sc = zero ? 1.f : amax / 448.f;
            if (tail)
                st16(crow + dim, u32x4{__float_as_uint(sc), 0u, 0u, 0u});
            else
                scales[row] = sc;
        }
    }
}

template <int XT>
__global__ __launch_bounds__(256) void quant_rows_kernel(int64_t rows, int dim, const void* x, uint8_t* codes,
                                                         int64_t cpitch, float* scales, int tail)
{
    quant_rows_body<XT>(rows, dim, x, codes, cpitch, scales, tail, blockIdx.x, gridDim.x);
}

// The two query preparations of an fp8 indexer with an fp8 MLA in one launch: blocks
// [0, g1) rotate and quantise the index queries, blocks [g1, grid) quantise the MLA
// queries (bf16 rows of mdim elements, codes packed, scales apart).
template <int DIM>
__global__ __launch_bounds__(256) void fp8_queries_kernel(int64_t rows, const void* x, uint8_t* codes, float* scales,
                                                          double inv_sqrt_dim, int g1, int64_t mrows, int mdim,
                                                          const void* mx, uint8_t* mcodes, float* mscales,
                                                          ClearWords clear)
{
    clear.run();
    if ((int)blockIdx.x < g1)
        rotate_quant_rows<DIM, kBF16>(rows, x, codes, scales, inv_sqrt_dim, RowMap{nullptr, 0, 0}, blockIdx.x, g1);
    else
        quant_rows_body<kBF16>(mrows, mdim, mx, mcodes, mdim, mscales, 0, blockIdx.x - g1, gridDim.x - g1);
}

template <int DIM>
hipError_t launch_dim(int64_t rows, const void* x, int xt, uint8_t* codes, float* scales, RowMap map, hipStream_t s,
                      ClearWords clear)
{
    const double inv = 1.0 / sqrt((double)DIM);
    constexpr int RPB = 4 * (64 / (DIM / 8));  // rows per block pass
    const dim3 grid((unsigned)std::min<int64_t>((rows + RPB - 1) / RPB, 8192));
    if (xt == kBF16)
        rotate_quant_kernel<DIM, kBF16><<<grid, 256, 0, s>>>(rows, x, codes, scales, inv, map, clear);
    else
        rotate_quant_kernel<DIM, kF32><<<grid, 256, 0, s>>>(rows, x, codes, scales, inv, map, clear);
    return hipGetLastError();
}

hipError_t launch_map(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, float* scales, RowMap map,
                      hipStream_t s, ClearWords clear = ClearWords{nullptr, 0})
{
    if (rows <= 0) return hipSuccess;
    switch (dim) {
        case 16: return launch_dim<16>(rows, x, x_dtype, codes, scales, map, s, clear);
        case 32: return launch_dim<32>(rows, x, x_dtype, codes, scales, map, s, clear);
        case 64: return launch_dim<64>(rows, x, x_dtype, codes, scales, map, s, clear);
        case 128: return launch_dim<128>(rows, x, x_dtype, codes, scales, map, s, clear);
        case 256: return launch_dim<256>(rows, x, x_dtype, codes, scales, map, s, clear);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_rotate_quant(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, float* scales,
                               hipStream_t s, uint32_t* zero, long long zero_words)
{
    return launch_map(rows, dim, x, x_dtype, codes, scales, RowMap{nullptr, 0, 0}, s, ClearWords{zero, zero_words});
}

hipError_t launch_quant_rows(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, int64_t cpitch,
                             float* scales, int tail, hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    if (dim <= 0 || dim % 16 != 0 || dim > 1024) return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>((rows + 3) / 4, 8192));
    if (x_dtype == kBF16)
        quant_rows_kernel<kBF16><<<grid, 256, 0, s>>>(rows, dim, x, codes, cpitch, scales, tail);
    else
        quant_rows_kernel<kF32><<<grid, 256, 0, s>>>(rows, dim, x, codes, cpitch, scales, tail);
    return hipGetLastError();
}

hipError_t launch_fp8_queries(int64_t rows, int dim, const void* x, uint8_t* codes, float* scales, int64_t mrows,
                              int mdim, const void* mx, uint8_t* mcodes, float* mscales, hipStream_t s,
                              uint32_t* zero, long long zero_words)
{
    if (dim != 128 || mdim <= 0 || mdim % 16 != 0 || mdim > 1024 || rows <= 0 || mrows <= 0) {
        const hipError_t e = launch_rotate_quant(rows, dim, x, kBF16, codes, scales, s, zero, zero_words);
        return e != hipSuccess ? e : launch_quant_rows(mrows, mdim, mx, kBF16, mcodes, mdim, mscales, 0, s);
    }
    constexpr int RPB = 4 * (64 / (128 / 8));  // index-query rows per block pass
    const int g1 = (int)std::min<int64_t>((rows + RPB - 1) / RPB, 8192);
    const int g2 = (int)std::min<int64_t>((mrows + 3) / 4, 8192);
    fp8_queries_kernel<128><<<dim3((unsigned)(g1 + g2)), 256, 0, s>>>(rows, x, codes, scales, 1.0 / sqrt(128.0), g1,
                                                                       mrows, mdim, mx, mcodes, mscales,
                                                                       ClearWords{zero, zero_words});
    return hipGetLastError();
}

hipError_t launch_cache_append(int batch, int t_new, int max_kv, int dim, const void* x, int x_dtype,
                               const int32_t* kv_len, uint8_t* codes, float* scales, hipStream_t s)
{
    return launch_map((int64_t)batch * t_new, dim, x, x_dtype, codes, scales, RowMap{kv_len, t_new, max_kv}, s);
}

}  // namespace dsa
