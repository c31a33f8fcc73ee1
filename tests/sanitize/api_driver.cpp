// api_driver.cpp -- the host side of the C ABI (nosa_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU: workspace
// queries over a grid of shapes, and every entry point with arguments its
// checks must reject.  The kernel launchers and the two HIP runtime calls the
// checks can reach are stubs here; a launcher stub aborts, so a call that
// got past its checks fails the run.  Built and run by tests/test_sanitize.py.
#include <cstdio>
#include <cstdlib>

#include "nosa_internal.h"

namespace nosa {
[[noreturn]] static void reached(const char* what)
{
    std::fprintf(stderr, "api driver: %s reached (a call passed its checks)\n", what);
    std::abort();
}
hipError_t launch_kc_build(const Plan&, const nosa_paged_kv&, const int32_t*, const int32_t*, int, hipStream_t)
{ reached("launch_kc_build"); }
hipError_t launch_scores_only(const Plan&, const nosa_paged_kv&, const nosa_bf16*, const int32_t*, const Workspace&,
                              float*, hipStream_t)
{ reached("launch_scores_only"); }
hipError_t launch_select(const Plan&, const int32_t*, const int32_t*, int, const float*, int32_t*, int32_t*,
                         hipStream_t)
{ reached("launch_select"); }
hipError_t launch_attend(const Plan&, const nosa_paged_kv&, const nosa_bf16*, const int32_t*, const int32_t*,
                         const int32_t*, const Workspace&, float*, float*, hipStream_t)
{ reached("launch_attend"); }
hipError_t launch_decode(const Plan&, const nosa_paged_kv&, const nosa_bf16*, const int32_t*, const Workspace&, float*,
                         float*, int32_t*, int32_t*, float*, hipStream_t, const Offload*)
{ reached("launch_decode"); }
hipError_t launch_pf_scores(const Plan&, const PfPlan&, const nosa_paged_kv&, const nosa_bf16*, const int32_t*,
                            const int32_t*, void*, float*, hipStream_t, const int32_t*)
{ reached("launch_pf_scores"); }
hipError_t launch_pf_attend(const Plan&, const PfPlan&, const nosa_paged_kv&, const nosa_bf16*, const int32_t*,
                            const int32_t*, const int32_t*, const int32_t*, float*, float*, hipStream_t,
                            const int32_t*)
{ reached("launch_pf_attend"); }
hipError_t launch_chunk_setup(const int32_t*, int, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t)
{ reached("launch_chunk_setup"); }
hipError_t launch_pack_qkv(int, int, int, const nosa_bf16*, nosa_bf16*, hipStream_t) { reached("launch_pack_qkv"); }
hipError_t launch_front(const Plan&, const nosa_paged_kv&, const nosa_bf16*, const nosa_bf16*, int, float,
                        const float*, const int32_t*, nosa_bf16*, hipStream_t)
{ reached("launch_front"); }
hipError_t static_scratch(void**) { reached("static_scratch"); }
hipError_t launch_check_inputs(const int32_t*, const int32_t*, const int32_t*, int, int, int, int, int, int32_t*,
                               hipStream_t)
{ reached("launch_check_inputs"); }
}  // namespace nosa

// no device: every pointer is "not device-readable host memory"
extern "C" hipError_t hipPointerGetAttributes(hipPointerAttribute_t*, const void*) { return hipErrorInvalidValue; }
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

static int failures = 0;
static void expect(bool ok, const char* what, int line)
{
    if (!ok) {
        std::fprintf(stderr, "api driver: line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

int main()
{
    EXPECT(nosa_abi_version() == NOSA_ABI_VERSION);
    for (int s = -1; s <= 7; ++s) EXPECT(nosa_status_string(static_cast<nosa_status>(s)) != nullptr);

    nosa_params p{16, 2, 128, 64, 32, 16, 64, 1024, 0.f, 0.f};
    const int heads[][2] = {{16, 2}, {32, 8}, {12, 3}, {8, 8}, {16, 1}};
    const int batches[] = {1, 8, 32, 1000};
    const int qlens[] = {1, 64, 2048};
    const int klens[] = {1, 4096, 131072, 524288};
    for (auto& h : heads)
        for (int B : batches)
            for (int Lq : qlens)
                for (int Lk : klens) {
                    nosa_params ph = p;
                    ph.num_q_heads = h[0];
                    ph.num_kv_heads = h[1];
                    size_t bytes = 0;
                    const nosa_status st = nosa_workspace_size(&ph, B, Lq, Lk, &bytes);
                    EXPECT(st == NOSA_OK || st == NOSA_ERR_UNSUPPORTED || st == NOSA_ERR_INVALID);
                    if (st == NOSA_OK) EXPECT(bytes > 0);
                    size_t pb = 0;
                    const nosa_status sp = nosa_prefill_sparse_workspace_size(&ph, B, Lk, 2048, &pb);
                    EXPECT(sp == NOSA_OK || sp == NOSA_ERR_UNSUPPORTED || sp == NOSA_ERR_INVALID);
                    size_t ob = 0;
                    const nosa_status so = nosa_offload_workspace_size(&ph, B, Lk, 128, &ob);
                    EXPECT(so == NOSA_OK || so == NOSA_ERR_UNSUPPORTED || so == NOSA_ERR_INVALID);
                }
    size_t bytes = 0;
    EXPECT(nosa_workspace_size(&p, 8, 1, 16384, &bytes) == NOSA_OK && bytes > 0);
    EXPECT(nosa_workspace_size(nullptr, 8, 1, 16384, &bytes) == NOSA_ERR_NULL);
    EXPECT(nosa_workspace_size(&p, 8, 1, 16384, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_workspace_size(&p, -1, 1, 16384, &bytes) != NOSA_OK);
    EXPECT(nosa_workspace_size(&p, 8, 1, -5, &bytes) != NOSA_OK);
    nosa_params bad = p;
    bad.num_kv_heads = 3;
    EXPECT(nosa_workspace_size(&bad, 8, 1, 16384, &bytes) == NOSA_ERR_INVALID);
    bad = p;
    bad.head_dim = 64;
    EXPECT(nosa_workspace_size(&bad, 8, 1, 16384, &bytes) != NOSA_OK);
    bad = p;
    bad.window = 1000;  // not a multiple of the block
    EXPECT(nosa_workspace_size(&bad, 8, 1, 16384, &bytes) != NOSA_OK);
    bad = p;
    bad.locality = 1.5f;
    EXPECT(nosa_workspace_size(&bad, 8, 1, 16384, &bytes) != NOSA_OK);
    EXPECT(nosa_prefill_sparse_workspace_size(&p, 1, 4096, 100, &bytes) != NOSA_OK);  // chunk not a multiple of 64
    EXPECT(nosa_offload_workspace_size(&p, 8, 16384, 0, &bytes) != NOSA_OK);
    EXPECT(nosa_offload_workspace_size(&p, 8, 16384, 100000, &bytes) != NOSA_OK);

    // entry points: fake device addresses are never dereferenced on the host,
    // and every call below must stop at its checks
    auto* fb = reinterpret_cast<nosa_bf16*>(0x10000);
    auto* fi = reinterpret_cast<int32_t*>(0x20000);
    auto* ff = reinterpret_cast<float*>(0x30000);
    void* ws = reinterpret_cast<void*>(0x40000);
    nosa_paged_kv kv{fb, fb, fb, fi, 256, 2048};
    nosa_paged_kv kv_null{nullptr, fb, fb, fi, 256, 2048};
    EXPECT(nosa_decode_step(nullptr, &kv, fb, fi, 8, 16384, ff, ff, fi, fi, ff, ws, 1 << 30, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_decode_step(&p, &kv_null, fb, fi, 8, 16384, ff, ff, fi, fi, ff, ws, 1 << 30, nullptr) ==
           NOSA_ERR_NULL);
    EXPECT(nosa_decode_step(&p, &kv, fb, fi, 8, 16384, ff, ff, fi, fi, ff, ws, 16, nullptr) == NOSA_ERR_WORKSPACE);
    EXPECT(nosa_decode_step(&p, &kv, fb, fi, 8, 16384, ff, ff, fi, fi, ff, nullptr, 1 << 30, nullptr) ==
           NOSA_ERR_WORKSPACE);
    EXPECT(nosa_decode_step(&bad, &kv, fb, fi, 8, 16384, ff, ff, fi, fi, ff, ws, 1 << 30, nullptr) != NOSA_OK);
    EXPECT(nosa_decode_step(&p, &kv, fb, fi, 8, 256 * 64 + 1, ff, ff, fi, fi, ff, ws, 1 << 30, nullptr) != NOSA_OK);
    EXPECT(nosa_decode_step_static(&p, &kv, fb, fi, 1000, 524288, ff, ff, fi, fi, ff, nullptr) != NOSA_OK);
    EXPECT(nosa_decode_step_static(&p, &kv, nullptr, fi, 8, 16384, ff, ff, fi, fi, ff, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_compress_keys(&p, &kv, nullptr, nullptr, 8, 16384, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_compress_keys(&p, &kv, fi, nullptr, -2, 16384, nullptr) != NOSA_OK);
    EXPECT(nosa_block_scores(&p, &kv, fb, fi, fi, 8, 2048, 16384, nullptr, ws, 1 << 30, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_block_scores(&p, &kv, fb, fi, fi, 8, 2048, 16384, ff, ws, 16, nullptr) == NOSA_ERR_WORKSPACE);
    EXPECT(nosa_select_blocks(&p, nullptr, fi, fi, 8, 2048, 16384, fi, fi, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_check_inputs(&p, &kv, nullptr, fi, 8, 1, 16384, nullptr, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_check_inputs(&p, nullptr, nullptr, fi, 8, 1, 16384, fi, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_check_inputs(&p, &kv, nullptr, fi, 8, 64, 16384, fi, nullptr) == NOSA_ERR_INVALID);
    EXPECT(nosa_check_inputs(&p, &kv, nullptr, fi, 8, 1, 256 * 64 + 1, fi, nullptr) == NOSA_ERR_INVALID);
    EXPECT(nosa_check_inputs(&bad, &kv, nullptr, fi, 8, 1, 16384, fi, nullptr) != NOSA_OK);
    EXPECT(nosa_select_blocks(&bad, ff, fi, fi, 8, 2048, 16384, fi, fi, nullptr) != NOSA_OK);
    EXPECT(nosa_sparse_attend(&p, &kv, fb, fi, fi, 8, 2048, 16384, fi, fi, nullptr, ff, ws, 1 << 30, nullptr) ==
           NOSA_ERR_NULL);
    EXPECT(nosa_sparse_attend(&p, &kv, fb, nullptr, fi, 8, 1, 16384, fi, fi, ff, ff, ws, 16, nullptr) ==
           NOSA_ERR_WORKSPACE);
    EXPECT(nosa_prefill_sparse(&p, &kv, fb, fi, 1, 4096, 100, ff, ff, ws, 1 << 30, nullptr) != NOSA_OK);
    EXPECT(nosa_prefill_sparse(&p, &kv, fb, fi, 1, 4096, 2048, ff, ff, ws, 16, nullptr) == NOSA_ERR_WORKSPACE);
    nosa_offload_kv okv{fb, fb, fb, fi, 256, 2048, fb, fb, 32, 128, fb, fb, fi, fi};
    // the host pages are not memory the device can read (no device here)
    EXPECT(nosa_offload_decode_step(&p, &okv, fb, fi, 8, 16384, ff, ff, fi, fi, nullptr, ws, 1 << 30, nullptr) !=
           NOSA_OK);
    EXPECT(nosa_offload_decode_step(&p, nullptr, fb, fi, 8, 16384, ff, ff, fi, fi, nullptr, ws, 1 << 30, nullptr) ==
           NOSA_ERR_NULL);
    EXPECT(nosa_pack_qkv_weights(&p, 0, fb, fb, nullptr) != NOSA_OK);
    EXPECT(nosa_pack_qkv_weights(&p, 2048, nullptr, fb, nullptr) == NOSA_ERR_NULL);
    nosa_front_params fr{2048, 0.f, nullptr};
    EXPECT(nosa_qkv_rope_append(&p, nullptr, &kv, fb, fb, fi, 8, 16384, fb, nullptr) == NOSA_ERR_NULL);
    EXPECT(nosa_layer_decode_step(&p, &fr, &kv, nullptr, fb, fi, 8, 16384, fb, ff, ff, fi, fi, ws, 1 << 30,
                                  nullptr) == NOSA_ERR_NULL);
    if (failures) return 1;
    std::printf("api driver: ok\n");
    return 0;
}
