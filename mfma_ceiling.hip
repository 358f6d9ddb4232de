// mfma_ceiling.hip -- sustained bf16 MFMA throughput, streaming-read bandwidth and
// random-row gather bandwidth of this GPU, for the roofline figures that bench.py reports beside the
// published peaks.
//
// Each wave issues back-to-back independent MFMAs (v_mfma_f32_32x32x16_bf16 or
// v_mfma_f32_16x16x32_bf16) for a fixed number of iterations, at two waves per
// SIMD, with operands that are either the same bits every time or drawn at
// random (uniform in [-1, 1]) and rotated so that every MFMA sees new bits, as
// real data does; the sustained rate depends on the operand values, not only on
// the instruction count.  The "vmix" cases follow every MFMA with n independent
// fma instructions (on small structured operands, in a fixed MFMA / VALU issue
// order) to measure how many other vector instructions an MFMA hides.  Only each
// thread's final sum is stored.  The "stream_read" cases read 1 GiB with a
// grid-stride loop of 16-byte loads (2048, 8192 or 32768 workgroups; 4 or 8 loads
// in flight per thread; plain or non-temporal loads) and store one sum per thread;
// the best of them is the streaming ceiling that the HBM-bound kernels are held to.  The "row_gather" cases
// read what the decode sparse MLA reads: rows of 1152 bytes (576 bf16) picked at
// random, without repetition, from each of 64 sequences of 32768 rows (a 2.4 GB
// latent cache), 2048 rows per sequence, 32 rows per tile, one 256-thread
// workgroup per (sequence, share of its rows), each 16-byte chunk loaded once,
// either into registers (two tiles in flight) or straight into LDS
// (global_load_lds_dwordx4, three tile buffers, two tiles in flight), with plain
// or non-temporal loads; three
// different row sets are rotated so that no launch finds the previous one's rows
// in the caches.  The best of them is the random-row gather ceiling.
// Prints one JSON line.
//
// Build and run (bench.py --mfma-ceiling does both):
//   hipcc --offload-arch=gfx950 -O3 -mllvm -amdgpu-mfma-vgpr-form=1 \
//         -Xclang -target-feature -Xclang -packed-fp32-ops -o mfma_ceiling mfma_ceiling.hip
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <utility>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kOps = 8;  // operand registers per lane per side (rotated)

// ops: [kOps][2][256 lanes] bf16x8 operand sets; the block's lanes read their own.
template <bool RANDOM>
__global__ __launch_bounds__(256, 2) void mfma32_kernel(const bf16x8* ops, float* out, int iters)
{
    bf16x8 a[kOps], b[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        a[i] = ops[(2 * i) * 256 + threadIdx.x];
        b[i] = ops[(2 * i + 1) * 256 + threadIdx.x];
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; it += kOps) {
#pragma unroll
        for (int u = 0; u < kOps; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 x = RANDOM ? a[(u + j) % kOps] : a[0];
                const bf16x8 y = RANDOM ? b[(3 * u + j) % kOps] : b[0];
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[j], 0, 0, 0);
            }
    }
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e) r += acc[j][e];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

template <bool RANDOM>
__global__ __launch_bounds__(256, 2) void mfma16_kernel(const bf16x8* ops, float* out, int iters)
{
    bf16x8 a[kOps], b[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        a[i] = ops[(2 * i) * 256 + threadIdx.x];
        b[i] = ops[(2 * i + 1) * 256 + threadIdx.x];
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; it += kOps) {
#pragma unroll
        for (int u = 0; u < kOps; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bf16x8 x = RANDOM ? a[(u + j) % kOps] : a[0];
                const bf16x8 y = RANDOM ? b[(3 * u + j) % kOps] : b[0];
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[j], 0, 0, 0);
            }
    }
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

// n fma instructions after every MFMA, in the order MFMA, n VALU, MFMA, ...
template <int NV>
__global__ __launch_bounds__(256, 2) void vmix16_kernel(const bf16x8* ops, float* out, int iters)
{
    (void)ops;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(threadIdx.x * 0.001f + i);
        b[i] = (__bf16)(1.f + i);
    }
    f32x4 acc[8];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        x[j] = threadIdx.x * 0.5f + j;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < NV; ++u) x[(j * NV + u) & 7] = fmaf(x[(j * NV + u) & 7], 0.999f, 1.f);
        }
        if constexpr (NV > 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
            }
        }
    }
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3] + x[j];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

template <int NV>
__global__ __launch_bounds__(256, 2) void vmix32_kernel(const bf16x8* ops, float* out, int iters)
{
    (void)ops;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(threadIdx.x * 0.001f + i);
        b[i] = (__bf16)(1.f + i);
    }
    f32x16 acc[4];
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = threadIdx.x * 0.5f + j;
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < NV; ++u) x[(j * NV + u) & 7] = fmaf(x[(j * NV + u) & 7], 0.999f, 1.f);
        }
        if constexpr (NV > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
            }
        }
    }
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e) r += acc[j][e];
#pragma unroll
    for (int j = 0; j < 8; ++j) r += x[j];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

// Sum of a 16-byte-aligned buffer of n4 float4 elements, U loads in flight per thread
// per iteration (non-temporal loads when NT); one partial sum per thread.
typedef float fv4 __attribute__((ext_vector_type(4)));
typedef unsigned uv4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 ld_f4(const float4* p)
{
    if constexpr (NT) {
        const fv4 v = __builtin_nontemporal_load(reinterpret_cast<const fv4*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const float4* p, size_t n4, float* out)
{
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    float acc = 0.f;
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld_f4<NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n4; i += stride) {
        const float4 a = ld_f4<NT>(p + i);
        acc += a.x + a.y + a.z + a.w;
    }
    out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Random-row gather (the access pattern of the decode sparse MLA).  Block w takes
// sequence w / nsplit and its share w % nsplit of the sequence's row list; a tile
// is 32 rows x 72 chunks of 16 bytes, chunk c = tid + 256 k (k < 9) being row
// c / 72, chunk c % 72.  Row offsets are 32-bit byte offsets from the sequence base.
constexpr int kGSeq = 64, kGRows = 32768, kGSel = 2048, kGRowB = 1152, kGCh = kGRowB / 16;
constexpr int kGTile = 32, kGTileCh = kGTile * kGCh, kGLoads = kGTileCh / 256;
static_assert(kGTileCh % 256 == 0, "tile chunks");

template <bool NT>
__global__ __launch_bounds__(256) void gather_reg_kernel(const char* cache, const int* rows, int nsplit,
                                                         unsigned* out)
{
    __shared__ unsigned roff[kGSel];
    const int seq = blockIdx.x / nsplit, part = blockIdx.x % nsplit;
    const int per = kGSel / nsplit, ntiles = per / kGTile;
    const char* base = cache + (size_t)seq * kGRows * kGRowB;
    for (int i = threadIdx.x; i < per; i += 256) roff[i] = (unsigned)rows[seq * kGSel + part * per + i] * kGRowB;
    __syncthreads();
    unsigned acc = 0;
    uint4 cur[kGLoads], nxt[kGLoads];
    auto load = [&](uint4(&d)[kGLoads], int t) {
#pragma unroll
        for (int k = 0; k < kGLoads; ++k) {
            const int c = threadIdx.x + 256 * k;
            const uint4* src = reinterpret_cast<const uint4*>(base + roff[t * kGTile + c / kGCh] + (c % kGCh) * 16);
            if constexpr (NT) {
                const uv4 v = __builtin_nontemporal_load(reinterpret_cast<const uv4*>(src));
                d[k] = make_uint4(v.x, v.y, v.z, v.w);
            } else {
                d[k] = *src;
            }
        }
    };
    load(cur, 0);
    for (int t = 0; t < ntiles; ++t) {
        load(nxt, t + 1 < ntiles ? t + 1 : t);  // unconditional: the wait covers this tile only
#pragma unroll
        for (int k = 0; k < kGLoads; ++k) {
            acc ^= cur[k].x ^ cur[k].y ^ cur[k].z ^ cur[k].w;
            cur[k] = nxt[k];
        }
    }
    out[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <bool NT>
__global__ __launch_bounds__(256) void gather_lds_kernel(const char* cache, const int* rows, int nsplit,
                                                         unsigned* out)
{
    __shared__ __attribute__((aligned(16))) uint4 buf[3 * kGTileCh];
    __shared__ unsigned roff[kGSel];
    const int seq = blockIdx.x / nsplit, part = blockIdx.x % nsplit;
    const int per = kGSel / nsplit, ntiles = per / kGTile;
    const char* base = cache + (size_t)seq * kGRows * kGRowB;
    for (int i = threadIdx.x; i < per; i += 256) roff[i] = (unsigned)rows[seq * kGSel + part * per + i] * kGRowB;
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    auto issue = [&](int t) {
        uint4* dst = buf + (t % 3) * kGTileCh;
#pragma unroll
        for (int k = 0; k < kGLoads; ++k) {
            const int c = threadIdx.x + 256 * k;
            const unsigned off = roff[t * kGTile + c / kGCh] + (c % kGCh) * 16;
            const unsigned lds = (unsigned)reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) uint4*)(dst + wave * 64 + 256 * k));
            if constexpr (NT)
                asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
            else
                asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
        }
    };
    unsigned acc = 0;
    issue(0);
    if (ntiles > 1) issue(1);
    for (int t = 0; t < ntiles; ++t) {
        // tile t has landed for every wave, and every wave is done with the buffer that
        // tile t + 2 refills
        if (t + 1 < ntiles)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(kGLoads) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
        if (t + 2 < ntiles) issue(t + 2);
        const uint4 v = buf[(t % 3) * kGTileCh + threadIdx.x];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    }
    out[blockIdx.x * 256 + threadIdx.x] = acc;
}

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

int main()
{
    const int blocks = 2048;  // 8 waves per CU over 256 CUs
    const int iters = 32768;  // ~15-25 ms per launch: long enough to reach the sustained clock
    std::vector<uint16_t> host(2 * kOps * 256 * 8);
    std::mt19937 rng(12345);
    std::uniform_real_distribution<float> uni(-1.f, 1.f);
    for (auto& h : host) {
        const float f = uni(rng);
        uint32_t u;
        std::memcpy(&u, &f, 4);
        h = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    bf16x8* ops = nullptr;
    float* out = nullptr;
    CHECK(hipMalloc(&ops, host.size() * 2));
    CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
    CHECK(hipMemcpy(ops, host.data(), host.size() * 2, hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    struct Case {
        const char* name;
        void (*k)(const bf16x8*, float*, int);
        double flop_per_iter_wave;
    } cases[] = {
        {"32x32x16_const", mfma32_kernel<false>, 4.0 * 32 * 32 * 16 * 2},
        {"32x32x16_random", mfma32_kernel<true>, 4.0 * 32 * 32 * 16 * 2},
        {"16x16x32_const", mfma16_kernel<false>, 8.0 * 16 * 16 * 32 * 2},
        {"16x16x32_random", mfma16_kernel<true>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_16x16x32_n0", vmix16_kernel<0>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_16x16x32_n2", vmix16_kernel<2>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_16x16x32_n3", vmix16_kernel<3>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_16x16x32_n4", vmix16_kernel<4>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_16x16x32_n6", vmix16_kernel<6>, 8.0 * 16 * 16 * 32 * 2},
        {"vmix_32x32x16_n0", vmix32_kernel<0>, 2.0 * 32 * 32 * 16 * 2},
        {"vmix_32x32x16_n3", vmix32_kernel<3>, 2.0 * 32 * 32 * 16 * 2},
        {"vmix_32x32x16_n6", vmix32_kernel<6>, 2.0 * 32 * 32 * 16 * 2},
        {"vmix_32x32x16_n9", vmix32_kernel<9>, 2.0 * 32 * 32 * 16 * 2},
    };
    printf("{\"probe\": \"sustained bf16 MFMA, streaming read\", \"blocks\": %d, \"waves_per_simd\": 2, \"iters\": %d, \"results\": {",
           blocks, iters);
    const int ncase = (int)(sizeof(cases) / sizeof(cases[0]));
    for (int c = 0; c < ncase; ++c) {
        cases[c].k<<<blocks, 256>>>(ops, out, iters);  // warm-up launch
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < 3; ++r) cases[c].k<<<blocks, 256>>>(ops, out, iters);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        ms /= 3;
        const double tflops = cases[c].flop_per_iter_wave * iters * 4.0 * blocks / (ms * 1e-3) / 1e12;
        printf("%s\"%s\": {\"ms\": %.3f, \"tflops\": %.1f, \"of_2516_tflops\": %.4f}", c ? ", " : "", cases[c].name,
               ms, tflops, tflops / 2516.6);
    }
    // streaming read of 1 GiB: grid sizes and loads in flight swept, the best is the ceiling
    const size_t n4 = (size_t)1 << 26;
    const int grids[3] = {2048, 8192, 32768};
    float4* big = nullptr;
    float* sums = nullptr;
    CHECK(hipMalloc(&big, n4 * sizeof(float4)));
    CHECK(hipMalloc(&sums, (size_t)grids[2] * 256 * sizeof(float)));
    CHECK(hipMemset(big, 0, n4 * sizeof(float4)));
    double best = 0.0;
    printf("}, \"stream_read\": {\"bytes\": %zu, \"cases\": {", n4 * sizeof(float4));
    for (int gi = 0; gi < 3; ++gi)
        for (int uu = 0; uu < 4; ++uu) {  // bit 0: 8 loads in flight instead of 4; bit 1: non-temporal
            auto launch = [&]() {
                switch (uu) {
                case 0: stream_read_kernel<4, false><<<grids[gi], 256>>>(big, n4, sums); break;
                case 1: stream_read_kernel<8, false><<<grids[gi], 256>>>(big, n4, sums); break;
                case 2: stream_read_kernel<4, true><<<grids[gi], 256>>>(big, n4, sums); break;
                default: stream_read_kernel<8, true><<<grids[gi], 256>>>(big, n4, sums); break;
                }
            };
            launch();  // warm-up launch
            CHECK(hipDeviceSynchronize());
            CHECK(hipEventRecord(e0));
            for (int r = 0; r < 10; ++r) launch();
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            ms /= 10;
            const double gbs = n4 * sizeof(float4) / (ms * 1e-3) / 1e9;
            best = gbs > best ? gbs : best;
            printf("%s\"grid%d_u%d%s\": {\"ms\": %.4f, \"GBs\": %.1f}", gi + uu ? ", " : "", grids[gi],
                   (uu & 1) ? 8 : 4, (uu & 2) ? "_nt" : "", ms, gbs);
        }
    printf("}, \"GBs\": %.1f}", best);
    CHECK(hipFree(sums));
    CHECK(hipFree(big));

    // random-row gather: three row sets, each 64 x 2048 distinct rows of 32768
    const size_t cache_bytes = (size_t)kGSeq * kGRows * kGRowB;
    char* cache = nullptr;
    int* rowsets = nullptr;
    unsigned* gout = nullptr;
    CHECK(hipMalloc(&cache, cache_bytes));
    CHECK(hipMemset(cache, 1, cache_bytes));
    CHECK(hipMalloc(&rowsets, 3 * (size_t)kGSeq * kGSel * sizeof(int)));
    CHECK(hipMalloc(&gout, (size_t)kGSeq * 16 * 256 * sizeof(unsigned)));
    {
        std::vector<int> perm(kGRows), h(3 * (size_t)kGSeq * kGSel);
        for (size_t sq = 0; sq < 3 * (size_t)kGSeq; ++sq) {
            for (int i = 0; i < kGRows; ++i) perm[i] = i;
            for (int i = 0; i < kGSel; ++i) {  // partial Fisher-Yates: the first kGSel of a random permutation
                const int j = i + (int)(rng() % (unsigned)(kGRows - i));
                std::swap(perm[i], perm[j]);
                h[sq * kGSel + i] = perm[i];
            }
        }
        CHECK(hipMemcpy(rowsets, h.data(), h.size() * sizeof(int), hipMemcpyHostToDevice));
    }
    const double gbytes = (double)kGSeq * kGSel * kGRowB;
    const int splits[2] = {4, 16};
    double gbest = 0.0;
    printf(", \"row_gather\": {\"bytes\": %.0f, \"row_bytes\": %d, \"cases\": {", gbytes, kGRowB);
    for (int path = 0; path < 4; ++path)  // bit 0: straight into LDS; bit 1: non-temporal
        for (int si = 0; si < 2; ++si) {
            const int ns = splits[si];
            auto launch = [&](int set) {
                const int* rs = rowsets + (size_t)set * kGSeq * kGSel;
                switch (path) {
                case 0: gather_reg_kernel<false><<<kGSeq * ns, 256>>>(cache, rs, ns, gout); break;
                case 1: gather_lds_kernel<false><<<kGSeq * ns, 256>>>(cache, rs, ns, gout); break;
                case 2: gather_reg_kernel<true><<<kGSeq * ns, 256>>>(cache, rs, ns, gout); break;
                default: gather_lds_kernel<true><<<kGSeq * ns, 256>>>(cache, rs, ns, gout); break;
                }
            };
            launch(0);  // warm-up launch
            CHECK(hipDeviceSynchronize());
            const int reps = 30;
            CHECK(hipEventRecord(e0));
            for (int r = 0; r < reps; ++r) launch(r % 3);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            ms /= reps;
            const double gbs = gbytes / (ms * 1e-3) / 1e9;
            gbest = gbs > gbest ? gbs : gbest;
            printf("%s\"%s%s_%dblocks\": {\"us\": %.2f, \"GBs\": %.1f}", path + si ? ", " : "",
                   (path & 1) ? "lds" : "registers", (path & 2) ? "_nt" : "", kGSeq * ns, ms * 1e3, gbs);
        }
    printf("}, \"GBs\": %.1f}}\n", gbest);
    CHECK(hipFree(gout));
    CHECK(hipFree(rowsets));
    CHECK(hipFree(cache));
    CHECK(hipFree(ops));
    CHECK(hipFree(out));
    return 0;
}
