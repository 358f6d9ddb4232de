// Host-side checks of the C ABI for the sanitizer build (tests/test_abi_sanitize.py):
// every workspace-size query over valid shapes, edge shapes and shapes near the
// int32 limits, and every entry point called with arguments that the host checks
// must reject (NULL, misaligned, bad sizes and dtypes, too small a workspace).
// No call here may reach a kernel launch: the pointers are stand-in addresses
// that are never dereferenced, so the program is safe with or without a GPU.
// Exit status 0 and "abi host checks ran" on success.
#include <dsa.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, int line)
{
    if (!ok) {
        std::fprintf(stderr, "check failed (line %d): %s\n", line, what);
        ++g_fail;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* const P16 = reinterpret_cast<void*>(uintptr_t{0x10000});   // 256-byte aligned stand-in
void* const P1 = reinterpret_cast<void*>(uintptr_t{0x10001});    // misaligned stand-in
void* const P4 = reinterpret_cast<void*>(uintptr_t{0x10004});    // 4- but not 16-byte aligned

dsa_shape base()
{
    dsa_shape s{};
    s.batch = 2;
    s.n_q = 4;
    s.max_kv = 256;
    s.idx_heads = 64;
    s.idx_dim = 128;
    s.topk = 64;
    s.heads = 128;
    s.qk_dim = 576;
    s.v_dim = 512;
    s.sm_scale = 0.07f;
    s.idx_dtype = DSA_BF16;
    s.mla_dtype = DSA_BF16;
    return s;
}

std::vector<dsa_shape> shapes()
{
    std::vector<dsa_shape> v;
    dsa_shape s = base();
    v.push_back(s);
    // the five workloads' shapes
    s = base(); s.batch = 1; s.n_q = 256; s.max_kv = 256; s.idx_dim = 64; s.idx_heads = 16; s.topk = 64;
    s.qk_dim = 80; s.v_dim = 64; s.heads = 16; s.idx_dtype = DSA_F32; s.mla_dtype = DSA_F32; v.push_back(s);
    s = base(); s.batch = 1; s.n_q = 4096; s.max_kv = 4096; s.topk = 2048; v.push_back(s);
    s = base(); s.batch = 64; s.n_q = 1; s.max_kv = 32768; s.topk = 2048; v.push_back(s);
    s = base(); s.batch = 1; s.n_q = 32768; s.max_kv = 32768; s.topk = 2048; v.push_back(s);
    s = base(); s.batch = 16; s.n_q = 1; s.max_kv = 131072; s.topk = 2048; s.idx_dtype = DSA_FP8_E4M3; v.push_back(s);
    s.mla_dtype = DSA_FP8_E4M3; v.push_back(s);
    // edges and near the int32 limits
    const int32_t big[] = {0, -1, 1, 2, 4095, 4096, 4097, (1 << 20), (1 << 20) + 1, INT_MAX / 2, INT_MAX, INT_MIN};
    for (int32_t x : big) {
        s = base(); s.batch = x; v.push_back(s);
        s = base(); s.n_q = x; s.max_kv = x > 0 ? x : 256; v.push_back(s);
        s = base(); s.max_kv = x; v.push_back(s);
        s = base(); s.topk = x; v.push_back(s);
        s = base(); s.heads = x; v.push_back(s);
        s = base(); s.idx_heads = x; v.push_back(s);
        s = base(); s.idx_dim = x; v.push_back(s);
        s = base(); s.qk_dim = x; v.push_back(s);
        s = base(); s.v_dim = x; v.push_back(s);
        s = base(); s.idx_dtype = x; v.push_back(s);
        s = base(); s.mla_dtype = x; v.push_back(s);
        s = base(); s.batch = x; s.n_q = x; s.max_kv = x; s.heads = x; v.push_back(s);
    }
    const float scales[] = {0.f, -1.f, INFINITY, -INFINITY, NAN, 1e-30f, 1e30f};
    for (float f : scales) {
        s = base(); s.sm_scale = f; v.push_back(s);
    }
    s = base(); s.n_q = 300; s.max_kv = 256; v.push_back(s);  // more queries than cache rows
    s = base(); s.batch = 4096; s.n_q = 4096; s.max_kv = 1 << 20; s.topk = 4096; v.push_back(s);
    s = base(); s.batch = 65536; s.n_q = 65536; s.max_kv = 65536; s.topk = 4096; s.heads = 4096; v.push_back(s);
    return v;
}

void sizes(const dsa_shape& s)
{
    // values are not checked here (the Python host tests do); the sanitizers watch
    // the arithmetic
    volatile size_t sink = 0;
    sink += dsa_forward_workspace_size(&s);
    sink += dsa_forward_min_workspace_size(&s);
    sink += dsa_topk_workspace_size(&s);
    sink += dsa_sparse_mla_workspace_size(&s);
    sink += dsa_index_topk_workspace_size(&s);
    sink += dsa_index_topk_min_workspace_size(&s);
    sink += dsa_sparse_mla_bwd_workspace_size(&s);
    sink += dsa_sparse_mla_bwd_min_workspace_size(&s);
    (void)sink;
}

// An error found on the host: not DSA_OK, and not DSA_ERR_HIP (which only a
// launch can return, and no call here may reach one).
bool rejected(dsa_status st) { return st != DSA_OK && st != DSA_ERR_HIP && st >= DSA_ERR_SCRATCH; }

// Entry points with arguments the host must reject, for one shape.
void rejects(const dsa_shape& s)
{
    const float* F = static_cast<const float*>(P16);
    const int32_t* I = static_cast<const int32_t*>(P16);
    float* Fo = static_cast<float*>(P16);
    int32_t* Io = static_cast<int32_t*>(P16);
    uint8_t* U = static_cast<uint8_t*>(P16);
    // NULL pointers
    EXPECT(rejected(dsa_index_scores(&s, nullptr, nullptr, F, P16, nullptr, I, Fo, nullptr)));
    EXPECT(rejected(dsa_topk(&s, nullptr, I, Io, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_sparse_mla_fwd(&s, nullptr, P16, I, I, P16, Fo, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_index_topk(&s, P16, nullptr, F, nullptr, nullptr, I, Io, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_sparse_mla_bwd(&s, P16, P16, I, I, F, nullptr, Fo, Fo, 0, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_forward(&s, nullptr, F, P16, nullptr, P16, P16, I, Io, P16, Fo, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_forward_noalloc(&s, nullptr, F, P16, nullptr, P16, P16, I, Io, P16, Fo, nullptr)));
    EXPECT(rejected(dsa_forward(nullptr, P16, F, P16, nullptr, P16, P16, I, Io, P16, Fo, P16, 1 << 20, nullptr)));
    // misaligned operands
    EXPECT(rejected(dsa_index_scores(&s, P1, nullptr, F, P16, nullptr, I, Fo, nullptr)));
    EXPECT(rejected(dsa_sparse_mla_fwd(&s, P4, P16, I, I, P16, Fo, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_forward(&s, P16, F, P16, nullptr, P16, P16, I, Io, P1, Fo, P16, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_forward(&s, P16, F, P16, nullptr, P16, P16, I, Io, P16, Fo, P4, 1 << 20, nullptr)));
    EXPECT(rejected(dsa_index_topk(&s, P16, nullptr, F, P16, nullptr, I, Io, P4, 1 << 20, nullptr)));
    // workspace missing or one byte short of the minimum
    EXPECT(rejected(dsa_forward(&s, P16, F, P16, nullptr, P16, P16, I, Io, P16, Fo, nullptr, 0, nullptr)));
    const size_t fmin = dsa_forward_min_workspace_size(&s);
    if (fmin > 0)
        EXPECT(rejected(dsa_forward(&s, P16, F, P16, nullptr, P16, P16, I, nullptr, P16, Fo, P16, fmin - 1, nullptr)));
    const size_t imin = dsa_index_topk_min_workspace_size(&s);
    if (imin > 0)
        EXPECT(rejected(dsa_index_topk(&s, P16, nullptr, F, P16, nullptr, I, Io, P16, imin - 1, nullptr)));
    const size_t bmin = dsa_sparse_mla_bwd_min_workspace_size(&s);
    if (bmin > 0)
        EXPECT(rejected(dsa_sparse_mla_bwd(&s, P16, P16, I, I, F, P16, Fo, Fo, 1, P16, bmin - 1, nullptr)));
    const size_t tws = dsa_topk_workspace_size(&s);
    if (tws > 0) EXPECT(rejected(dsa_topk(&s, F, I, Io, P16, tws - 1, nullptr)));
    // row-wise entry points: bad sizes, dtypes, pointers
    EXPECT(rejected(dsa_rotate_quant_fp8(0, 128, P16, DSA_BF16, U, Fo, nullptr)));
    EXPECT(rejected(dsa_rotate_quant_fp8(-5, 128, P16, DSA_BF16, U, Fo, nullptr)));
    EXPECT(rejected(dsa_rotate_quant_fp8(8, 100, P16, DSA_BF16, U, Fo, nullptr)));
    EXPECT(rejected(dsa_rotate_quant_fp8(8, 128, P16, DSA_FP8_E4M3, U, Fo, nullptr)));
    EXPECT(rejected(dsa_rotate_quant_fp8(8, 128, P1, DSA_BF16, U, Fo, nullptr)));
    EXPECT(rejected(dsa_rotate_quant_fp8(INT64_MAX, INT_MAX, P16, DSA_BF16, U, Fo, nullptr)));
    EXPECT(rejected(dsa_index_cache_append_fp8(0, 1, 16, 128, P16, DSA_BF16, I, U, Fo, nullptr)));
    EXPECT(rejected(dsa_index_cache_append_fp8(2, 1, 16, 129, P16, DSA_BF16, I, U, Fo, nullptr)));
    EXPECT(rejected(dsa_index_cache_append_fp8(2, 1, 16, 128, nullptr, DSA_BF16, I, U, Fo, nullptr)));
    EXPECT(rejected(dsa_index_cache_append_fp8(INT_MAX, INT_MAX, INT_MAX, 256, P16, 7, I, U, Fo, nullptr)));
    EXPECT(rejected(dsa_mla_kv_quant_fp8(0, 576, P16, DSA_BF16, U, nullptr)));
    EXPECT(rejected(dsa_mla_kv_quant_fp8(4, 577, P16, DSA_BF16, U, nullptr)));
    EXPECT(rejected(dsa_mla_kv_quant_fp8(4, 4096, P16, DSA_BF16, U, nullptr)));
    EXPECT(rejected(dsa_mla_kv_quant_fp8(4, 576, P16, DSA_BF16, nullptr, nullptr)));
}

}  // namespace

int main()
{
    for (int st = -12; st <= 3; ++st) EXPECT(dsa_status_string(static_cast<dsa_status>(st)) != nullptr);
    const std::vector<dsa_shape> v = shapes();
    for (const dsa_shape& s : v) {
        sizes(s);
        rejects(s);
    }
    EXPECT(dsa_forward_workspace_size(nullptr) == 0);
    EXPECT(dsa_topk_workspace_size(nullptr) == 0);
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("abi host checks ran: %zu shapes\n", v.size());
    return 0;
}
