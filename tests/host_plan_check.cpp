// Host-only checks of the merge's validator, layout adapter and chunk planner.
// Built with g++ (no HIP) under AddressSanitizer and UBSan by
// tests/test_abi_host.py; links context_lse_merge_amd/csrc/dcp_host.cpp only.
// Device pointers here are made-up, suitably aligned integers: nothing is
// dereferenced and nothing is launched.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dcp_internal.h"

static int g_failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);   \
            ++g_failures;                                                    \
        }                                                                    \
    } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
    void* stream = fake(0x5000);
    dcp_workspace* ws = nullptr;
    CHECK(dcp_workspace_create(128, 16, 4, 512, DCP_DTYPE_BF16, stream, &ws) == DCP_OK);
    CHECK(ws != nullptr);

    const int64_t B = 500, H = 64, D = 512;
    const uintptr_t attn = 0x10000000, lse = 0x20000000, out = 0x30000000, out_lse = 0x40000000;
    dcp::MergePlan plan;

    // Contiguous [B, 64, 512] attention, BHC LSE [B, 16, 4], contiguous out.
    int rc = dcp::plan_merge(ws, fake(attn), B, H, H * D, D, reinterpret_cast<const float*>(lse), DCP_LSE_BHC,
                             16 * 4, 4, 1, DCP_LSE_BASE_E, fake(out), 16 * D, D, reinterpret_cast<float*>(out_lse),
                             16, stream, &plan);
    CHECK(rc == DCP_OK);
    CHECK(plan.n_chunks == 4);  // ceil(500 / 128)
    CHECK(plan.chunk == 128);
    CHECK(plan.args.a_sb == H * D && plan.args.a_sj == D && plan.args.a_ss == 16 * D);  // shard s at head s*16 + j
    CHECK(plan.args.l_sb == 64 && plan.args.l_sj == 4 && plan.args.l_ss == 1);
    CHECK(plan.args.cp == 4 && plan.args.h_local == 16);
    CHECK(plan.args.to_log2 > 1.4426f && plan.args.to_log2 < 1.4427f);
    for (int64_t k = 0; k < plan.n_chunks; ++k) {
        dcp::MergeArgs a = dcp::chunk_args(plan, k);
        const int64_t t0 = k * 128, t1 = (t0 + 128 < B) ? t0 + 128 : B;
        CHECK(reinterpret_cast<uintptr_t>(a.attn) == attn + 2 * t0 * H * D);
        CHECK(reinterpret_cast<uintptr_t>(a.lse) == lse + 4 * t0 * 64);
        CHECK(reinterpret_cast<uintptr_t>(a.out) == out + 2 * t0 * 16 * D);
        CHECK(reinterpret_cast<uintptr_t>(a.out_lse) == out_lse + 4 * t0 * 16);
        CHECK(a.rows == (t1 - t0) * 16);
    }

    // FlashMLA [B, H, 1] LSE: shard stride is h_local * l1; base 2 constants are 1.
    rc = dcp::plan_merge(ws, fake(attn), B, H, H * D, D, reinterpret_cast<const float*>(lse), DCP_LSE_BH1, 64, 1, 0,
                         DCP_LSE_BASE_2, fake(out), 16 * D, D, nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK);
    CHECK(plan.args.l_sj == 1 && plan.args.l_ss == 16 && plan.args.out_lse == nullptr);
    CHECK(plan.args.to_log2 == 1.0f && plan.args.from_log2 == 1.0f);

    // 24 heads viewed out of a 128-head backing buffer (padded token stride).
    dcp_workspace* ws6 = nullptr;
    CHECK(dcp_workspace_create(8, 6, 4, 512, DCP_DTYPE_BF16, stream, &ws6) == DCP_OK);
    rc = dcp::plan_merge(ws6, fake(attn), 5, 24, 128 * D, D, reinterpret_cast<const float*>(lse), DCP_LSE_BH1, 24, 1,
                         0, DCP_LSE_BASE_E, fake(out), 6 * D, D, nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK && plan.n_chunks == 1 && plan.args.rows == 30 && plan.args.a_ss == 6 * D);

    // A capacity above the per-launch token limit is split further: 70000
    // tokens with capacity 100000 run as 65535 + 4465.
    dcp_workspace* wsw = nullptr;
    CHECK(dcp_workspace_create(100000, 16, 4, 512, DCP_DTYPE_BF16, stream, &wsw) == DCP_OK);
    const uintptr_t wattn = uintptr_t{1} << 44, wlse = uintptr_t{2} << 44, wout = uintptr_t{3} << 44;
    rc = dcp::plan_merge(wsw, fake(wattn), 70000, H, H * D, D, reinterpret_cast<const float*>(wlse), DCP_LSE_BHC,
                         16 * 4, 4, 1, DCP_LSE_BASE_E, fake(wout), 16 * D, D, nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK && plan.chunk == dcp::kMaxLaunchTokens && plan.n_chunks == 2);
    CHECK(plan.args.rows == 65535 * 16 && dcp::chunk_args(plan, 1).rows == 4465 * 16);
    CHECK(reinterpret_cast<uintptr_t>(dcp::chunk_args(plan, 1).attn) == wattn + 2 * int64_t{65535} * H * D);
    CHECK(dcp_workspace_destroy(wsw) == DCP_OK);

    // B == 0 is a no-op plan.
    rc = dcp::plan_merge(ws, nullptr, 0, H, 0, 0, nullptr, DCP_LSE_BHC, 0, 0, 0, DCP_LSE_BASE_E, nullptr, 0, 0,
                         nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK && plan.n_chunks == 0);

    // Every check fires before anything could be launched.
    auto call = [&](const dcp_workspace* w, const void* at, int64_t b, int h, int64_t sb, int64_t sh, uintptr_t l,
                    int layout, int64_t l0, int64_t l1, int64_t l2, int mode, void* o, int64_t osb, int64_t osh,
                    uintptr_t ol, int64_t olsb, void* st) {
        return dcp::plan_merge(w, at, b, h, sb, sh, reinterpret_cast<const float*>(l), layout, l0, l1, l2, mode, o,
                               osb, osh, reinterpret_cast<float*>(ol), olsb, st, &plan);
    };
    const int64_t sb = H * D, sh = D;
    CHECK(call(nullptr, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_WORKSPACE);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, fake(0x6000)) ==
          DCP_ERR_STREAM);
    CHECK(std::strstr(dcp_last_error(), "stream") != nullptr);
    CHECK(call(ws, fake(attn), -1, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);
    CHECK(call(ws, fake(attn), 4, 62, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);
    CHECK(call(ws, fake(attn), 4, 32, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_WORKSPACE);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 7, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 9, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);
    CHECK(call(ws, nullptr, 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);
    CHECK(call(ws, fake(attn), 4, 64, -sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_LAYOUT);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D / 2, 0, 0, stream) ==
          DCP_ERR_LAYOUT);  // out rows overlap
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, out_lse, 8, stream) ==
          DCP_ERR_LAYOUT);  // out_lse rows overlap
    CHECK(call(ws, fake(attn + 8), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_ALIGN);
    CHECK(call(ws, fake(attn), 4, 64, sb + 4, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_ALIGN);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse + 2, 0, 64, 4, 1, 0, fake(out), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_ALIGN);
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(attn + 2 * D), 16 * D, D, 0, 0, stream) ==
          DCP_ERR_INVALID_ARG);  // out inside attn
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), 16 * D, D, lse + 16, 16, stream) ==
          DCP_ERR_INVALID_ARG);  // out_lse inside lse
    // A transposed but non-overlapping out ([h_local, B, D] storage) is fine.
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), D, 4 * D, 0, 0, stream) == DCP_OK);

    // Workspace creation errors.
    dcp_workspace* bad = nullptr;
    CHECK(dcp_workspace_create(0, 16, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG && bad == nullptr);
    CHECK(dcp_workspace_create(8, 0, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(8, 16, 65, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(8, 16, 4, 256, 0, stream, &bad) == DCP_ERR_LAYOUT);
    CHECK(dcp_workspace_create(8, 16, 4, 512, 3, stream, &bad) == DCP_ERR_LAYOUT);
    CHECK(dcp_workspace_create(8, 16, 4, 512, 0, stream, nullptr) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(int64_t{1} << 27, 16, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);

    CHECK(dcp_workspace_destroy(ws) == DCP_OK);
    CHECK(dcp_workspace_destroy(ws6) == DCP_OK);
    CHECK(dcp_workspace_destroy(nullptr) == DCP_OK);
    CHECK(std::strcmp(dcp_status_string(DCP_ERR_ALIGN), "DCP_ERR_ALIGN") == 0);

    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host plan checks passed\n");
    return 0;
}
