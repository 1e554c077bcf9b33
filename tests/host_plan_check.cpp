// Host-only checks of the merge's validator, layout adapter and chunk planner.
// Built with g++ (no HIP) under AddressSanitizer and UBSan by
// tests/test_abi_host.py; links context_lse_merge_amd/csrc/dcp_host.cpp only.
// Device pointers here are made-up, suitably aligned integers: nothing is
// dereferenced and nothing is launched.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

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

// The variable-length work plan, run sequentially with the planning kernel's
// arithmetic, against the capacities varlen_layout gives the scratch: the
// list fits, the slots fit, every pair's tiles are covered once by splits of
// at most st tiles, and the list runs longest split first.
static void check_varlen_plan(const std::vector<int64_t>& lens, int hq, int64_t T, int cp, bool il) {
    const int64_t B = static_cast<int64_t>(lens.size());
    const dcp::VarlenLayout lay = dcp::varlen_layout(B, hq, T, cp);
    const int rbt = (hq + dcp::kMlaRowsPerBlock - 1) / dcp::kMlaRowsPerBlock;
    int64_t total = 0;
    for (int64_t L : lens)
        for (int s = 0; s < cp; ++s) total += rbt * dcp::varlen_shard_tiles(L < 0 ? 0 : (L > T ? T : L), s, cp, il);
    const int64_t st = dcp::varlen_split_tiles(total);
    CHECK(st >= dcp::kMlaMinSplitTiles && st * dcp::kVarlenTarget >= total);
    int64_t items = 0, slots = 0, split_pairs = 0, covered = 0;
    std::vector<int64_t> bins(dcp::kMlaPlanThreads, 0);
    for (int64_t L : lens) {
        const int64_t Lc = L < 0 ? 0 : (L > T ? T : L);
        int64_t keys = 0;
        for (int s = 0; s < cp; ++s) {
            const int64_t t = dcp::varlen_shard_tiles(Lc, s, cp, il);
            keys += t;
            const int64_t n = dcp::varlen_splits(t, st);
            CHECK(n >= 1 && (n - 1) * st < t + (t == 0) && n * st >= t);
            for (int64_t p = 0; p < n; ++p) {
                const int64_t size = (p + 1) * st < t ? st : t - p * st;
                CHECK(size >= 0 && size <= st && (size > 0 || t == 0));
                ++bins[dcp::varlen_bin(size, st)];
                covered += size;
            }
            items += rbt * n;
            if (n > 1) {
                slots += rbt * n;
                split_pairs += rbt;
            }
        }
        // Every key of the token is in exactly one shard.
        CHECK(keys * dcp::kMlaKeysPerTile >= Lc && (keys - cp) * dcp::kMlaKeysPerTile < Lc + 1);
    }
    CHECK(covered * rbt == total);
    CHECK(items <= lay.items);
    CHECK(slots <= lay.slots);
    CHECK(split_pairs < dcp::kVarlenTarget || split_pairs == 0);
    CHECK(bins[dcp::kMlaPlanThreads - 1] == 0 || dcp::varlen_bin(st, st) == dcp::kMlaPlanThreads - 1);
    CHECK(lay.pairs == B * rbt * cp && lay.items == lay.pairs + dcp::kVarlenTarget);
    CHECK(lay.off_hdr % 64 == 0 && lay.off_items % 16 == 0 && lay.off_split % 16 == 0);
    CHECK(lay.bytes == lay.off_split + dcp::kVarlenTarget * sizeof(dcp::VarlenSplit));
    // fp16 partial rows, then one LSE and one scale per row, then the plan.
    const size_t rows = static_cast<size_t>(lay.slots) * dcp::kMlaRowsPerBlock;
    CHECK(lay.off_lse == rows * dcp::kMlaVDim * 2 && lay.off_scale == lay.off_lse + rows * 4);
    CHECK(lay.off_hdr >= lay.off_scale + rows * 4);
}

// The fixed-length producer's split scratch: fp16 rows [B][nsplit*cp*hq][512],
// then part_lse and part_scale [B][nsplit*cp*hq], and the merge over splits
// reading them as a scaled-fp16 payload.
static void fixed_split_checks() {
    const int64_t B = 3, T = 131072;
    const int hq = 128, cp = 4;
    int32_t nsplit;
    int64_t split_len;
    size_t need;
    dcp::mla_split(B, hq, T, cp, &nsplit, &split_len, &need);
    CHECK(nsplit > 1);
    const int64_t heads = static_cast<int64_t>(nsplit) * cp * hq;
    CHECK(need == static_cast<size_t>(B * heads) * (dcp::kMlaVDim * 2 + 8));
    const uintptr_t q = uintptr_t{1} << 40, kv = uintptr_t{2} << 40, o = uintptr_t{3} << 40,
                    l = uintptr_t{4} << 40, scr = uintptr_t{6} << 40;
    dcp::MlaPlan plan;
    CHECK(dcp::plan_mla(fake(q), B, hq, hq * 576, 576, fake(kv), T, 576, nullptr, DCP_DTYPE_BF16, cp, 0.07f,
                        DCP_LSE_BASE_E, fake(o), cp * hq * 512, 512, reinterpret_cast<float*>(l), cp * hq, fake(scr),
                        need, &plan) == DCP_OK);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_o) == scr);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_lse) == scr + B * heads * dcp::kMlaVDim * 2);
    CHECK(plan.args.part_scale == plan.args.part_lse + B * heads);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_scale + B * heads) == scr + need);
    CHECK(plan.reduce.in_dtype == dcp::kPayloadF16Scaled && plan.reduce.sc_off == B * heads);
    CHECK(plan.reduce.attn == plan.args.part_o && plan.reduce.lse == plan.args.part_lse);
    CHECK(plan.reduce.cp == nsplit && plan.reduce.h_local == cp * hq && plan.reduce.a_sb == heads * dcp::kMlaVDim);
    CHECK(!plan.deep);  // three row blocks share each key range: the one-tile-ahead loop
    CHECK(dcp::plan_mla(fake(q), B, hq, hq * 576, 576, fake(kv), T, 576, nullptr, DCP_DTYPE_BF16, cp, 0.07f,
                        DCP_LSE_BASE_E, fake(o), cp * hq * 512, 512, reinterpret_cast<float*>(l), cp * hq, fake(scr),
                        need - 1, &plan) == DCP_ERR_WORKSPACE);
    // One row block (B * hq <= 128): two tiles in flight; two row blocks: one tile ahead.
    const struct { int64_t B; int hq; bool deep; } rb[] = {{1, 128, true}, {3, 40, true}, {1, 1, true},
                                                           {2, 128, false}, {1, 160, false}, {129, 1, false}};
    for (const auto& c : rb) {
        size_t n;
        dcp::mla_split(c.B, c.hq, T, cp, &nsplit, &split_len, &n);
        CHECK(dcp::plan_mla(fake(q), c.B, c.hq, c.hq * 576, 576, fake(kv), T, 576, nullptr, DCP_DTYPE_BF16, cp, 0.07f,
                            DCP_LSE_BASE_E, fake(o), cp * c.hq * 512, 512, reinterpret_cast<float*>(l), cp * c.hq,
                            fake(scr), n, &plan) == DCP_OK);
        CHECK(plan.deep == c.deep);
    }
}

// dcp_mla_decode_merged: the counters first, the split partials after them;
// EPILOGUE marks the plan fused (no separate split reduction or shard
// merge), NONE, REDUCTIONS and AUTO plan the shard merge over (o_part,
// lse_part) in the FlashMLA layout, REDUCTIONS and AUTO as part of the
// combined reduction launch where the keys are split and cp <= 16; errors
// before anything could run.
static void merged_plan_checks() {
    const int64_t B = 3, T = 131072;
    const int hq = 128, cp = 4;
    int32_t nsplit;
    int64_t split_len;
    size_t part;
    dcp::mla_split(B, hq, T, cp, &nsplit, &split_len, &part);
    const size_t cnt = dcp::merged_counter_bytes(B, hq, cp);
    CHECK(cnt == 256 && nsplit > 1);  // 3 row blocks x (4 + 1) counters, rounded to 256 bytes
    size_t need = 0;
    CHECK(dcp_mla_decode_merged_scratch_size(B, hq, T, cp, &need) == DCP_OK && need == cnt + part);
    const uintptr_t q = uintptr_t{1} << 40, kv = uintptr_t{2} << 40, o = uintptr_t{3} << 40,
                    l = uintptr_t{4} << 40, out = uintptr_t{5} << 40, scr = uintptr_t{6} << 40,
                    ol = uintptr_t{7} << 40;
    auto plan_it = [&](int fuse, size_t bytes, uintptr_t out_p, dcp::MlaPlan* plan) {
        return dcp::plan_mla_merged(fake(q), B, hq, hq * 576, 576, fake(kv), T, 576, DCP_DTYPE_BF16, cp, 0.07f,
                                    DCP_LSE_BASE_2, fake(o), cp * hq * 512, 512, reinterpret_cast<float*>(l),
                                    cp * hq, fake(out_p), hq * 512, 512, reinterpret_cast<float*>(ol), hq, fuse,
                                    fake(scr), bytes, plan);
    };
    dcp::MlaPlan plan;
    CHECK(plan_it(DCP_FUSE_EPILOGUE, need, out, &plan) == DCP_OK);
    CHECK(plan.args.fused == 1 && !plan.merge_shards);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.split_cnt) == scr);
    CHECK(plan.args.rb_cnt == plan.args.split_cnt + 3 * cp);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_o) == scr + cnt);
    CHECK(plan.args.to_log2 == 1.0f && plan.args.from_log2 == 1.0f);
    for (int fuse : {DCP_FUSE_NONE, DCP_FUSE_REDUCTIONS, DCP_FUSE_AUTO}) {
        CHECK(plan_it(fuse, need, out, &plan) == DCP_OK);
        CHECK(plan.args.fused == 0 && plan.merge_shards);
        CHECK(plan.reduce_merge == (fuse == DCP_FUSE_REDUCTIONS || (fuse == DCP_FUSE_AUTO && nsplit >= 16)));
        const dcp::MergeArgs& m = plan.shard_merge;
        CHECK(m.attn == fake(o) && m.a_sb == cp * hq * 512 && m.a_sj == 512 && m.a_ss == hq * 512);
        CHECK(m.l_sb == cp * hq && m.l_sj == 1 && m.l_ss == hq && m.h_local == hq && m.cp == cp);
        CHECK(reinterpret_cast<uintptr_t>(m.out) == out && m.o_sb == hq * 512 && m.o_sj == 512 && m.cached == 1);
    }
    CHECK(plan_it(DCP_FUSE_EPILOGUE, need - 1, out, &plan) == DCP_ERR_WORKSPACE);
    CHECK(std::strstr(dcp_last_error(), "dcp_mla_decode_merged_scratch_size") != nullptr);
    CHECK(plan_it(4, need, out, &plan) == DCP_ERR_INVALID_ARG);
    // The combined launch is not taken with one split per shard, nor above 16 shards.
    for (const int64_t Bx : {int64_t{64}, int64_t{3}}) {
        const int cpx = Bx == 3 ? 32 : 4;
        int32_t nx;
        int64_t lx;
        size_t px;
        dcp::mla_split(Bx, hq, T, cpx, &nx, &lx, &px);
        CHECK((Bx == 64) == (nx == 1));
        size_t needx = 0;
        CHECK(dcp_mla_decode_merged_scratch_size(Bx, hq, T, cpx, &needx) == DCP_OK);
        for (int fuse : {DCP_FUSE_REDUCTIONS, DCP_FUSE_AUTO}) {
            CHECK(dcp::plan_mla_merged(fake(q), Bx, hq, hq * 576, 576, fake(kv), T, 576, DCP_DTYPE_BF16, cpx, 0.07f,
                                       DCP_LSE_BASE_2, fake(o), cpx * hq * 512, 512, reinterpret_cast<float*>(l),
                                       cpx * hq, fake(out), hq * 512, 512, reinterpret_cast<float*>(ol), hq, fuse,
                                       fake(scr), needx, &plan) == DCP_OK);
            CHECK(plan.merge_shards && !plan.reduce_merge);
        }
    }
    CHECK(plan_it(DCP_FUSE_NONE, need, o + 1024, &plan) == DCP_ERR_INVALID_ARG);    // out inside o_part
    CHECK(plan_it(DCP_FUSE_NONE, need, scr + 4096, &plan) == DCP_ERR_INVALID_ARG);  // out inside the scratch
    CHECK(plan_it(DCP_FUSE_NONE, need, out + 8, &plan) == DCP_ERR_ALIGN);
}

// The plan's 32-bit shard sizes against their plain 64-bit definition.
static void shard_formula_checks() {
    std::mt19937_64 rng(7);
    for (int trial = 0; trial < 200000; ++trial) {
        const int32_t cp = 1 + static_cast<int32_t>(rng() % 64);
        const int32_t s = static_cast<int32_t>(rng() % cp);
        const int64_t L = (trial % 2) ? static_cast<int64_t>(rng() % 5000)
                                      : static_cast<int64_t>(rng() % (int64_t{dcp::kVarlenMaxLen} + 1));
        const int64_t n_c = ((s + 1) * L) / cp - (s * L) / cp;
        const int64_t n_i = L > s ? (L - s + cp - 1) / cp : 0;
        CHECK(dcp::varlen_shard_tiles(static_cast<int32_t>(L), s, cp, false) == (n_c + 31) / 32);
        CHECK(dcp::varlen_shard_tiles(static_cast<int32_t>(L), s, cp, true) == (n_i + 31) / 32);
    }
    // Size bins: 0 for an empty split, the top bin for a full one, monotone in between.
    for (int32_t st : {8, 9, 100, 549, 4096, 1 << 20, dcp::kVarlenMaxLen}) {
        CHECK(dcp::varlen_bin(0, st) == 0);
        CHECK(dcp::varlen_bin(st, st) == dcp::kMlaPlanThreads - 1);
        int prev = 0;
        for (int32_t k = 1; k <= 64; ++k) {
            const int32_t size = static_cast<int32_t>((static_cast<int64_t>(st) * k) / 64);
            const int b = dcp::varlen_bin(size, st);
            CHECK(b >= prev && b < dcp::kMlaPlanThreads);
            prev = b;
        }
    }
    CHECK(dcp::varlen_split_tiles(int64_t{1} << 50) == dcp::kVarlenMaxLen);
}

static void varlen_plan_checks() {
    shard_formula_checks();
    std::mt19937_64 rng(20261202);
    const int64_t T = 131072;
    for (int trial = 0; trial < 200; ++trial) {
        const int64_t B = 1 + static_cast<int64_t>(rng() % 300);
        const int cp = 1 + static_cast<int>(rng() % 8);
        const int hq = (trial % 3 == 0) ? 200 : 128;
        std::vector<int64_t> lens(B);
        for (auto& L : lens) {
            switch (trial % 4) {
                case 0: L = 1 + static_cast<int64_t>(rng() % T); break;             // uniform
                case 1: L = T; break;                                               // all full
                case 2: L = (rng() % 10 == 0) ? T : static_cast<int64_t>(rng() % 4096);  // skewed
                default: L = static_cast<int64_t>(rng() % 600) - 100;               // short, some clamped
            }
        }
        check_varlen_plan(lens, hq, T, cp, trial % 2 == 0);
    }
    check_varlen_plan({T}, 128, T, 4, true);           // one long token: many splits per pair
    check_varlen_plan({0, 0, 0}, 16, T, 4, false);     // nothing to attend to
    check_varlen_plan({5}, 16, 0, 1, false);           // max_seq_len 0
    CHECK(dcp::varlen_layout(4, 16, 100, 4).slots == 0);  // no pair can exceed 8 tiles

    // Scratch size query and the plan's pointers into the scratch.
    size_t bytes = 0;
    CHECK(dcp_mla_partial_decode_varlen_scratch_size(64, 128, T, 4, &bytes) == DCP_OK);
    CHECK(bytes == dcp::varlen_layout(64, 128, T, 4).bytes);
    CHECK(dcp_mla_partial_decode_varlen_scratch_size(0, 128, T, 4, &bytes) == DCP_OK && bytes == 0);
    const uintptr_t q = uintptr_t{1} << 40, kv = uintptr_t{2} << 40, o = uintptr_t{3} << 40,
                    l = uintptr_t{4} << 40, seq = uintptr_t{5} << 40, scr = uintptr_t{6} << 40;
    const dcp::VarlenLayout lay = dcp::varlen_layout(64, 128, T, 4);
    const dcp::MlaVarlen vl{reinterpret_cast<const int32_t*>(seq), 0, DCP_KV_INTERLEAVED};
    dcp::MlaPlan plan;
    CHECK(dcp::plan_mla(fake(q), 64, 128, 128 * 576, 576, fake(kv), T, 576, &vl, DCP_DTYPE_BF16, 4, 0.07f,
                        DCP_LSE_BASE_E, fake(o), 512 * 512, 512, reinterpret_cast<float*>(l), 512, fake(scr),
                        lay.bytes, &plan) == DCP_OK);
    CHECK(plan.varlen && plan.blocks == lay.items && plan.args.slots == lay.slots);
    CHECK(!plan.deep);  // the variable-length decode always runs the one-tile-ahead loop
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_lse) == scr + lay.off_lse);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.part_scale) == scr + lay.off_scale);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.vl_hdr) == scr + lay.off_hdr);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.vl_items) == scr + lay.off_items);
    CHECK(reinterpret_cast<uintptr_t>(plan.args.vl_splits) == scr + lay.off_split);
    CHECK(dcp::plan_mla(fake(q), 64, 128, 128 * 576, 576, fake(kv), T, 576, &vl, DCP_DTYPE_BF16, 4, 0.07f,
                        DCP_LSE_BASE_E, fake(o), 512 * 512, 512, reinterpret_cast<float*>(l), 512, fake(scr),
                        lay.bytes - 1, &plan) == DCP_ERR_WORKSPACE);
}

// A fake, 256-byte aligned device address for workspace buffers (never dereferenced).
constexpr uintptr_t kWsBuf = uintptr_t{0x7} << 40;

size_t ws_bytes(int64_t capacity, int h_local, int cp) {
    size_t n = 0;
    CHECK(dcp_workspace_size(capacity, h_local, cp, 512, DCP_DTYPE_BF16, &n) == DCP_OK);
    return n;
}

int main() {
    void* stream = fake(0x5000);
    dcp_workspace* ws = nullptr;
    CHECK(dcp_workspace_create(fake(kWsBuf), ws_bytes(128, 16, 4), 128, 16, 4, 512, DCP_DTYPE_BF16, stream, &ws) ==
          DCP_OK);
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
    CHECK(dcp_workspace_create(fake(kWsBuf), ws_bytes(8, 6, 4), 8, 6, 4, 512, DCP_DTYPE_BF16, stream, &ws6) == DCP_OK);
    rc = dcp::plan_merge(ws6, fake(attn), 5, 24, 128 * D, D, reinterpret_cast<const float*>(lse), DCP_LSE_BH1, 24, 1,
                         0, DCP_LSE_BASE_E, fake(out), 6 * D, D, nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK && plan.n_chunks == 1 && plan.args.rows == 30 && plan.args.a_ss == 6 * D);

    // A capacity above the per-launch token limit is split further: 70000
    // tokens with capacity 100000 run as 65535 + 4465.
    dcp_workspace* wsw = nullptr;
    CHECK(dcp_workspace_create(fake(kWsBuf), ws_bytes(100000, 16, 4), 100000, 16, 4, 512, DCP_DTYPE_BF16, stream,
                               &wsw) == DCP_OK);
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
    // Strides the kernel cannot take as 32-bit values are rejected.
    CHECK(call(ws, fake(attn), 2, 64, int64_t{1} << 31, sh, lse, 0, 64, 4, 1, 0, fake(uintptr_t{1} << 45), 16 * D, D,
               0, 0, stream) == DCP_ERR_LAYOUT);
    CHECK(call(ws, fake(attn), 2, 64, (int64_t{1} << 31) - 8, sh, lse, 0, 64, 4, 1, 0, fake(uintptr_t{1} << 45),
               16 * D, D, 0, 0, stream) == DCP_OK);
    CHECK(call(ws, fake(attn), 2, 64, sb, sh, lse, 0, int64_t{1} << 31, 4, 1, 0, fake(uintptr_t{1} << 45), 16 * D,
               D, 0, 0, stream) == DCP_ERR_LAYOUT);
    // A transposed but non-overlapping out ([h_local, B, D] storage) is fine.
    CHECK(call(ws, fake(attn), 4, 64, sb, sh, lse, 0, 64, 4, 1, 0, fake(out), D, 4 * D, 0, 0, stream) == DCP_OK);

    // Workspace creation errors.
    dcp_workspace* bad = nullptr;
    void* wb = fake(kWsBuf);
    const size_t big = size_t{1} << 40;
    CHECK(dcp_workspace_create(wb, big, 0, 16, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG && bad == nullptr);
    CHECK(dcp_workspace_create(wb, big, 8, 0, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(wb, big, 8, 16, 65, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(wb, big, 8, 16, 4, 256, 0, stream, &bad) == DCP_ERR_LAYOUT);
    CHECK(dcp_workspace_create(wb, big, 8, 16, 4, 512, 3, stream, &bad) == DCP_ERR_LAYOUT);
    CHECK(dcp_workspace_create(wb, big, 8, 16, 4, 512, 0, stream, nullptr) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(wb, big, int64_t{1} << 27, 16, 4, 512, 0, stream, &bad) == DCP_ERR_INVALID_ARG);
    // The device buffer: its size, too small or missing, misaligned.
    size_t need = 0;
    CHECK(dcp_workspace_size(8, 16, 4, 512, 0, &need) == DCP_OK);
    CHECK(need == size_t{8} * 16 * 4 * 1024 + size_t{8} * 16 * 4 * 4);  // both regions already multiples of 256
    CHECK(dcp_workspace_size(3, 5, 3, 512, 1, &need) == DCP_OK);
    CHECK(need == (size_t{45} * 1024 + 255) / 256 * 256 + (size_t{45} * 4 + 255) / 256 * 256);
    CHECK(dcp_workspace_size(0, 16, 4, 512, 0, &need) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_size(8, 16, 4, 512, 0, nullptr) == DCP_ERR_INVALID_ARG);
    CHECK(dcp_workspace_create(wb, ws_bytes(8, 16, 4) - 1, 8, 16, 4, 512, 0, stream, &bad) == DCP_ERR_WORKSPACE &&
          bad == nullptr);
    CHECK(std::strstr(dcp_last_error(), "dcp_workspace_size") != nullptr);
    CHECK(dcp_workspace_create(nullptr, big, 8, 16, 4, 512, 0, stream, &bad) == DCP_ERR_WORKSPACE);
    CHECK(dcp_workspace_create(fake(kWsBuf + 8), big, 8, 16, 4, 512, 0, stream, &bad) == DCP_ERR_ALIGN);
    // The landing zone: [capacity, H, D] payload at the buffer's start, the [capacity, H] LSEs after it.
    dcp_workspace* wz = nullptr;
    CHECK(dcp_workspace_create(fake(kWsBuf), ws_bytes(3, 5, 3), 3, 5, 3, 512, 0, stream, &wz) == DCP_OK);
    void* ra = nullptr;
    float* rl = nullptr;
    int64_t rsb = 0, rsh = 0, rlsb = 0;
    CHECK(dcp_workspace_recv(wz, &ra, &rsb, &rsh, &rl, &rlsb) == DCP_OK);
    CHECK(reinterpret_cast<uintptr_t>(ra) == kWsBuf && rsb == 15 * 512 && rsh == 512 && rlsb == 15);
    CHECK(reinterpret_cast<uintptr_t>(rl) == kWsBuf + (45 * 1024 + 255) / 256 * 256);
    CHECK(dcp_workspace_recv(wz, &ra, &rsb, nullptr, &rl, &rlsb) == DCP_ERR_INVALID_ARG);
    // A staged merge over the landing zone plans like any other.
    rc = dcp::plan_merge(wz, ra, 3, 15, rsb, rsh, rl, DCP_LSE_BH1, rlsb, 1, 0, DCP_LSE_BASE_E, fake(out), 5 * D, D,
                         nullptr, 0, stream, &plan);
    CHECK(rc == DCP_OK && plan.args.a_ss == 5 * D && plan.args.l_ss == 5 && plan.n_chunks == 1);
    CHECK(dcp_workspace_destroy(wz) == DCP_OK);
    CHECK(dcp_workspace_recv(nullptr, &ra, &rsb, &rsh, &rl, &rlsb) == DCP_ERR_WORKSPACE);

    CHECK(dcp_workspace_destroy(ws) == DCP_OK);
    CHECK(dcp_workspace_destroy(ws6) == DCP_OK);
    CHECK(dcp_workspace_destroy(nullptr) == DCP_OK);
    CHECK(std::strcmp(dcp_status_string(DCP_ERR_ALIGN), "DCP_ERR_ALIGN") == 0);

    varlen_plan_checks();
    fixed_split_checks();
    merged_plan_checks();

    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host plan checks passed\n");
    return 0;
}
