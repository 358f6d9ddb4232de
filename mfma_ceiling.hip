// mfma_ceiling.hip -- sustained bf16 MFMA throughput of this GPU, for the
// roofline figures that bench.py reports against the published peak.
//
// Each wave issues back-to-back independent MFMAs (v_mfma_f32_32x32x16_bf16 or
// v_mfma_f32_16x16x32_bf16) for a fixed number of iterations, at two waves per
// SIMD, with operands that are either the same bits every time or drawn at
// random (uniform in [-1, 1]) and rotated so that every MFMA sees new bits, as
// real data does.  The matrix units draw more power on changing operands, so the
// clock, and with it the sustained rate, is lower for the second kind.  Only each
// thread's final sum is stored.  Prints one JSON line.
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
    };
    printf("{\"probe\": \"sustained bf16 MFMA\", \"blocks\": %d, \"waves_per_simd\": 2, \"iters\": %d, \"results\": {",
           blocks, iters);
    for (int c = 0; c < 4; ++c) {
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
    printf("}}\n");
    CHECK(hipFree(ops));
    CHECK(hipFree(out));
    return 0;
}
