// quant.hip -- Hadamard rotation + e4m3 quantisation of indexer operands.
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
// One wave per row.  The transform is the in-place butterfly, carried in fp64
// so that its only rounding before the final fp32 is the 1/sqrt(dim) scaling;
// the fp32 divisions are correctly rounded.  e4m3 (OCP E4M3FN: bias 7, max 448,
// no infinities) is encoded from the fp32 bit pattern with round-half-even.
#include "dsa_common.h"
#include "dsa_kernels.h"

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

template <int DIM, int XT>
__global__ __launch_bounds__(256) void rotate_quant_kernel(int64_t rows, const void* x, uint8_t* codes,
                                                           float* scales, double inv_sqrt_dim, RowMap map)
{
    constexpr int E = DIM >= 64 ? DIM / 64 : 1;   // elements per lane: index e*64 + lane
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t orow = map(row);
    if (orow < 0) return;
    double v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * 64 + lane;
        float xv = 0.f;
        if (i < DIM) {
            if constexpr (XT == kBF16)
                xv = bf16_to_f32(((const uint16_t*)x)[row * DIM + i]);
            else
                xv = ((const float*)x)[row * DIM + i];
        }
        v[e] = (double)xv;
    }
    // butterfly over every bit of the element index
#pragma unroll
    for (int h = 1; h < DIM; h <<= 1) {
        if (h < 64) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double o = __shfl_xor(v[e], h, 64);
                v[e] = (lane & h) ? (o - v[e]) : (v[e] + o);
            }
        } else {
            const int he = h / 64;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (e & he) continue;
                const double a0 = v[e], b0 = v[e + he];
                v[e] = a0 + b0;
                v[e + he] = a0 - b0;
            }
        }
    }
    float xf[E];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool live = e * 64 + lane < DIM;
        xf[e] = (float)(v[e] * inv_sqrt_dim);
        if (live) amax = fmaxf(amax, fabsf(xf[e]));
    }
    amax = wave_max(amax);
    const bool zero = amax == 0.f;
    const float r = zero ? 0.f : 448.f / amax;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * 64 + lane;
        if (i < DIM) codes[orow * DIM + i] = zero ? (uint8_t)0 : e4m3_encode(xf[e] * r);
    }
    if (lane == 0) scales[orow] = zero ? 1.f : amax / 448.f;
}

template <int DIM>
hipError_t launch_dim(int64_t rows, const void* x, int xt, uint8_t* codes, float* scales, RowMap map, hipStream_t s)
{
    const double inv = 1.0 / sqrt((double)DIM);
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (xt == kBF16)
        rotate_quant_kernel<DIM, kBF16><<<grid, 256, 0, s>>>(rows, x, codes, scales, inv, map);
    else
        rotate_quant_kernel<DIM, kF32><<<grid, 256, 0, s>>>(rows, x, codes, scales, inv, map);
    return hipGetLastError();
}

hipError_t launch_map(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, float* scales, RowMap map,
                      hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    switch (dim) {
        case 16: return launch_dim<16>(rows, x, x_dtype, codes, scales, map, s);
        case 32: return launch_dim<32>(rows, x, x_dtype, codes, scales, map, s);
        case 64: return launch_dim<64>(rows, x, x_dtype, codes, scales, map, s);
        case 128: return launch_dim<128>(rows, x, x_dtype, codes, scales, map, s);
        case 256: return launch_dim<256>(rows, x, x_dtype, codes, scales, map, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_rotate_quant(int64_t rows, int dim, const void* x, int x_dtype, uint8_t* codes, float* scales,
                               hipStream_t s)
{
    return launch_map(rows, dim, x, x_dtype, codes, scales, RowMap{nullptr, 0, 0}, s);
}

hipError_t launch_cache_append(int batch, int t_new, int max_kv, int dim, const void* x, int x_dtype,
                               const int32_t* kv_len, uint8_t* codes, float* scales, hipStream_t s)
{
    return launch_map((int64_t)batch * t_new, dim, x, x_dtype, codes, scales, RowMap{kv_len, t_new, max_kv}, s);
}

}  // namespace dsa
