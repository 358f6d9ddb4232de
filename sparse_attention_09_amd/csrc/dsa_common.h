// dsa_common.h -- device helpers shared by the gfx950 kernels of the DSA path.
//
// MFMA lane layouts used throughout (wave64; checked on the hardware):
//   v_mfma_f32_16x16x32_bf16 / _16x16x32_fp8_fp8 / _16x16x4f32
//     A (16 x K): lane l holds row l%16, k-block l/16 (8, 8 or 1 elements)
//     B (K x 16): lane l holds column l%16, the same k-block
//     C (16 x 16): lane l holds column l%16, rows 4*(l/16) + 0..3
// Because a product sums over k, any fixed assignment of the contraction index
// to (k-block, slot) works as long as A and B use the same one; the kernels
// use that freedom to choose which 16-byte chunks of a row each lane loads.
//
// ds_read_b64_tr_b16 (gfx950): inside every 16-lane group, lane i receives
// element j (j = 0..3) from the address supplied by lane 4*j + i/4 of its group,
// at 16-bit offset i%4.  Handing it rows of a row-major tile gives a lane the
// column-wise (contraction-major) operand of a value matrix.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum DType : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 16-byte global load / store through plain vector accesses.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// The same with the non-temporal hint, for data that one access reads or writes once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }

// Raw buffer accesses (no stride) through a descriptor whose record count bounds
// them: a load at or past the end returns zero, a store there is dropped, with no
// branch.  Offsets are bytes (32-bit: the library's supported sizes, L_max <= 2^20
// rows of at most 512 bytes, keep every offset below 2^31); kDropOffset lies past
// every record count used.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kDropOffset = 0x7FFFFFF0;

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(buf_rsrc r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(buf_rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ void buf_st4(buf_rsrc r, int off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0); }
__device__ __forceinline__ void buf_st8(buf_rsrc r, int off, uint32_t lo, uint32_t hi)
{
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, off, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(u32x2 a, u32x2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c,
                                                      0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 first.
__device__ __forceinline__ uint32_t float_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Sum / max over the four 16-lane groups (lanes l, l^16, l^32, l^48), on the
// gfx950 row swaps instead of LDS permutes: v_permlane16_swap of a register
// with itself leaves rows (r0, r0, r2, r2) in one copy and (r1, r1, r3, r3) in
// the other, v_permlane32_swap does the same for row pairs.  The pairing of the
// additions is that of the xor-16-then-xor-32 shuffle sum.
__device__ __forceinline__ float group4_sum(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ float group4_max(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

}  // namespace dsa
