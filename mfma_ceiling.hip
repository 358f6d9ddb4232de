// mfma_ceiling.hip -- sustained bf16 MFMA throughput and streaming-read bandwidth
// of this GPU, for the roofline figures that bench.py reports beside the
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
// in flight per thread) and store one sum per thread; the best of them is the plain
// streaming ceiling that the HBM-bound kernels are held to.
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
// per iteration; one partial sum per thread.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const float4* p, size_t n4, float* out)
{
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    float acc = 0.f;
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n4; i += stride) {
        const float4 a = p[i];
        acc += a.x + a.y + a.z + a.w;
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
        for (int uu = 0; uu < 2; ++uu) {
            auto launch = [&]() {
                if (uu == 0)
                    stream_read_kernel<4><<<grids[gi], 256>>>(big, n4, sums);
                else
                    stream_read_kernel<8><<<grids[gi], 256>>>(big, n4, sums);
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
            printf("%s\"grid%d_u%d\": {\"ms\": %.4f, \"GBs\": %.1f}", gi + uu ? ", " : "", grids[gi], uu ? 8 : 4,
                   ms, gbs);
        }
    printf("}, \"GBs\": %.1f}}\n", best);
    CHECK(hipFree(sums));
    CHECK(hipFree(big));
    CHECK(hipFree(ops));
    CHECK(hipFree(out));
    return 0;
}
