// dcp_host.cpp -- argument validation, the strided-view layout adapter and the
// ordered chunk planner of the DCP LSE merge, plus the workspace object and
// error reporting.  Pure host C++: no HIP call, no device access.
//
// Layout adapter ("[DCP] Run fi_a2a on FlashInfer's fused all-to-all + LSE
// reduce", sglang PR #40539, Modifications): the [B, H, D] attention output is
// viewed as [B, H/cp, cp, D] without a copy, head h belonging to shard
// h / (H/cp); so element (b, j, s, d) sits at b*sb + (s*H_local + j)*sh + d,
// i.e. local-head stride sh and shard stride H_local*sh.  The LSE is either
// [B, H/cp, cp] or FlashMLA's [B, H, 1] (PR #40539, Accuracy Tests); the
// latter is the same view with shard stride H_local*l1.
//
// Chunk planner (PR #40539, Modifications and Coordination): batches wider
// than the workspace run as several launches over consecutive token ranges,
// in order, on the workspace's stream.  A call on any other stream is rejected
// before anything is enqueued (PR #40539, Accuracy Tests: a call from a third
// stream is refused before any exchange starts).
//
// Input checks: the later text of PR #40539 drops the copy of strided or
// misaligned partials and lets the kernel check its inputs; here an input the
// kernel cannot read directly is rejected with an error, never copied.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "dcp_internal.h"

namespace dcp {

namespace {
thread_local char g_error[512] = "";

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte range [lo, hi) covered by a strided 2-D set of rows:
// n1 x n2 rows of `row_elems` elements of `elem` bytes, row (i, k) at
// base + i*s1 + k*s2 (elements).  Strides are non-negative here.
struct Extent {
    uintptr_t lo, hi;
};
Extent extent(const void* base, int64_t n1, int64_t s1, int64_t n2, int64_t s2, int64_t row_elems, size_t elem) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    int64_t last = (n1 - 1) * s1 + (n2 - 1) * s2 + row_elems;
    return Extent{lo, lo + static_cast<uintptr_t>(last) * elem};
}
bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// Rows of `row` elements at offsets i*s1 + k*s2 (0 <= i < n1, 0 <= k < n2)
// are pairwise disjoint if, with the strides sorted, the small one clears a
// row and the big one clears a full run of the small one.
bool rows_disjoint(int64_t n1, int64_t s1, int64_t n2, int64_t s2, int64_t row) {
    if (n1 <= 1) return n2 <= 1 || s2 >= row;
    if (n2 <= 1) return s1 >= row;
    int64_t ns = n1, ss = s1, sb = s2;  // the smaller stride, its count, and the bigger stride
    if (s2 < s1) {
        ns = n2; ss = s2; sb = s1;
    }
    return ss >= row && sb >= (ns - 1) * ss + row;
}
}  // namespace

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_error[0] = '\0';
    return DCP_OK;
}

int plan_merge(const dcp_workspace* ws, const void* attn, int64_t B, int H, int64_t attn_sb, int64_t attn_sh,
               const float* lse, int lse_layout, int64_t l0, int64_t l1, int64_t l2, int lse_mode, void* out,
               int64_t out_sb, int64_t out_sh, float* out_lse, int64_t out_lse_sb, void* hip_stream,
               MergePlan* plan) {
    if (!ws || ws->magic != kWorkspaceMagic)
        return fail(DCP_ERR_WORKSPACE, "dcp_lse_combine: no valid workspace (create one with dcp_workspace_create)");
    if (hip_stream != ws->stream)
        return fail(DCP_ERR_STREAM,
                    "dcp_lse_combine: called on stream %p but the workspace serves stream %p; a workspace serves "
                    "one ordered stream, create another workspace for this stream",
                    hip_stream, ws->stream);
    const int cp = ws->cp, h_local = ws->h_local;
    if (B < 0) return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: B = %lld is negative", (long long)B);
    if (H <= 0 || H % cp != 0)
        return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: H = %d is not a positive multiple of cp = %d", H, cp);
    if (H / cp != h_local)
        return fail(DCP_ERR_WORKSPACE,
                    "dcp_lse_combine: H / cp = %d local heads but the workspace was created for h_local = %d", H / cp,
                    h_local);
    if (lse_layout != DCP_LSE_BHC && lse_layout != DCP_LSE_BH1)
        return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: lse_layout %d is neither DCP_LSE_BHC nor DCP_LSE_BH1",
                    lse_layout);
    if (lse_mode != DCP_LSE_BASE_E && lse_mode != DCP_LSE_BASE_2)
        return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: lse_mode %d is neither DCP_LSE_BASE_E nor DCP_LSE_BASE_2",
                    lse_mode);
    if (B == 0) {
        *plan = MergePlan{};
        return ok();
    }
    if (!attn || !lse || !out)
        return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: attn, lse and out must be non-null when B > 0");

    const int64_t D = ws->d;
    if (attn_sb < 0 || attn_sh < 0 || l0 < 0 || l1 < 0 || out_sb < 0 || out_sh < 0 || out_lse_sb < 0 ||
        (lse_layout == DCP_LSE_BHC && l2 < 0))
        return fail(DCP_ERR_LAYOUT, "dcp_lse_combine: strides must be non-negative");
    if (!rows_disjoint(B, out_sb, h_local, out_sh, D))
        return fail(DCP_ERR_LAYOUT,
                    "dcp_lse_combine: out rows overlap (out_sb = %lld, out_sh = %lld, D = %lld): each of the "
                    "B x h_local output rows needs D elements of its own",
                    (long long)out_sb, (long long)out_sh, (long long)D);
    if (out_lse && !rows_disjoint(B, out_lse_sb, h_local, 1, 1))
        return fail(DCP_ERR_LAYOUT, "dcp_lse_combine: out_lse_sb = %lld < h_local = %d makes out_lse rows overlap",
                    (long long)out_lse_sb, h_local);

    if (!aligned(attn, 16) || !aligned(out, 16))
        return fail(DCP_ERR_ALIGN, "dcp_lse_combine: attn (%p) and out (%p) must be 16-byte aligned", attn, out);
    if (attn_sb % 8 || attn_sh % 8 || out_sb % 8 || out_sh % 8)
        return fail(DCP_ERR_ALIGN,
                    "dcp_lse_combine: attn_sb, attn_sh, out_sb and out_sh must be multiples of 8 elements "
                    "(16 bytes); got %lld, %lld, %lld, %lld",
                    (long long)attn_sb, (long long)attn_sh, (long long)out_sb, (long long)out_sh);
    if (!aligned(lse, 4) || (out_lse && !aligned(out_lse, 4)))
        return fail(DCP_ERR_ALIGN, "dcp_lse_combine: lse and out_lse must be 4-byte aligned");

    // Layout adapter: (b, j, s) strides of O and of the LSE.
    MergeArgs a{};
    a.attn = attn;
    a.in_dtype = ws->dtype;
    a.cached = ws->load_policy == DCP_LOAD_CACHED ? 1 : 0;
    a.lse = lse;
    a.out = static_cast<uint16_t*>(out);
    a.out_lse = out_lse;
    a.a_sb = attn_sb;
    a.a_sj = attn_sh;
    a.a_ss = static_cast<int64_t>(h_local) * attn_sh;
    a.l_sb = l0;
    if (lse_layout == DCP_LSE_BHC) {
        a.l_sj = l1;
        a.l_ss = l2;
    } else {
        a.l_sj = l1;
        a.l_ss = static_cast<int64_t>(h_local) * l1;
    }
    a.o_sb = out_sb;
    a.o_sj = out_sh;
    a.ol_sb = out_lse_sb;
    a.h_local = h_local;
    a.cp = cp;
    a.dtype = ws->dtype;
    if (lse_mode == DCP_LSE_BASE_2) {
        a.to_log2 = 1.0f;
        a.from_log2 = 1.0f;
    } else {
        a.to_log2 = 1.4426950408889634f;  // log2 e
        a.from_log2 = 0.6931471805599453f; // ln 2
    }

    // Outputs may not overlap inputs or each other.
    const Extent e_attn = extent(attn, B, attn_sb, H, attn_sh, D, 2);
    const Extent e_out = extent(out, B, out_sb, h_local, out_sh, D, 2);
    int64_t lse_last;
    if (lse_layout == DCP_LSE_BHC)
        lse_last = (B - 1) * l0 + (h_local - 1) * l1 + (cp - 1) * l2 + 1;
    else
        lse_last = (B - 1) * l0 + (H - 1) * l1 + 1;
    const Extent e_lse{reinterpret_cast<uintptr_t>(lse),
                       reinterpret_cast<uintptr_t>(lse) + static_cast<uintptr_t>(lse_last) * 4};
    if (overlaps(e_out, e_attn) || overlaps(e_out, e_lse))
        return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: out overlaps attn or lse; the merge is out of place");
    if (out_lse) {
        const Extent e_ol = extent(out_lse, B, out_lse_sb, 1, 0, h_local, 4);
        if (overlaps(e_ol, e_attn) || overlaps(e_ol, e_lse) || overlaps(e_ol, e_out))
            return fail(DCP_ERR_INVALID_ARG, "dcp_lse_combine: out_lse overlaps attn, lse or out");
    }

    if (!merge_strides_fit(a))
        return fail(DCP_ERR_LAYOUT,
                    "dcp_lse_combine: attn and lse strides must be below 2^31 elements (attn_sb = %lld, attn_sh = %lld, "
                    "lse strides %lld, %lld, %lld)",
                    (long long)attn_sb, (long long)attn_sh, (long long)l0, (long long)l1, (long long)l2);

    plan->args = a;
    plan->B = B;
    // Tokens are the second grid dimension, which holds at most kMaxLaunchTokens
    // blocks: a wider capacity is split further.  Chunks give the same bits
    // as one launch, so the extra split is invisible to the caller.
    plan->chunk = ws->capacity < kMaxLaunchTokens ? ws->capacity : kMaxLaunchTokens;
    plan->n_chunks = (B + plan->chunk - 1) / plan->chunk;
    plan->args.rows = static_cast<int32_t>((B < plan->chunk ? B : plan->chunk) * h_local);
    return ok();
}

MergeArgs merge_args_at(const MergeArgs& a0, int64_t t0, int64_t tokens) {
    MergeArgs a = a0;
    a.attn = static_cast<const char*>(a.attn) + t0 * a.a_sb * payload_bytes(a.in_dtype);
    a.lse += t0 * a.l_sb;
    a.out += t0 * a.o_sb;
    if (a.out_lse) a.out_lse += t0 * a.ol_sb;
    a.rows = static_cast<int32_t>(tokens * a.h_local);
    return a;
}

MergeArgs chunk_args(const MergePlan& plan, int64_t k) {
    const int64_t t0 = k * plan.chunk;
    const int64_t t1 = (t0 + plan.chunk < plan.B) ? t0 + plan.chunk : plan.B;
    return merge_args_at(plan.args, t0, t1 - t0);
}

// ------------------------------------------------------------- MLA decode plan
//
// Split-KV: with B*hq query rows in workgroups of 128 and cp shards there are
// ceil(B*hq/128)*cp units of work -- 4 at B = 1 with 128 heads and cp = 4, far
// too few for 256 compute units.  Each shard's keys are therefore split into
// nsplit ranges processed by separate workgroups; each leaves a normalised
// partial (fp16 rows scaled by a power of two) and its LSE, and the merge
// kernel reduces the splits exactly as it merges DCP shards.  The split count aims at about kMlaTargetBlocks
// workgroups and never gives a split fewer than kMlaMinSplitKeys keys.  Every
// token has the same T keys here, so the host decides; with per-token
// lengths the planning kernel does (varlen_layout sizes its scratch).

void mla_split(int64_t B, int hq, int64_t T, int cp, int32_t* nsplit, int64_t* split_len, size_t* scratch_bytes) {
    const int64_t rows = B * hq;
    const int64_t row_blocks = (rows + kMlaRowsPerBlock - 1) / kMlaRowsPerBlock;
    const int64_t shard_max = (T + cp - 1) / cp;  // longest shard
    int64_t n = 1;
    if (row_blocks > 0 && shard_max > 0) {
        const int64_t base = row_blocks * cp;
        n = (kMlaTargetBlocks + base - 1) / base;
        const int64_t n_max = (shard_max + kMlaMinSplitKeys - 1) / kMlaMinSplitKeys;
        if (n > n_max) n = n_max;
        if (n > kMlaMaxSplits) n = kMlaMaxSplits;
        if (n < 1) n = 1;
    }
    int64_t len = (shard_max + n - 1) / n;
    len = ((len + kMlaKeysPerTile - 1) / kMlaKeysPerTile) * kMlaKeysPerTile;
    if (len < kMlaKeysPerTile) len = kMlaKeysPerTile;
    if (shard_max > 0) n = (shard_max + len - 1) / len;  // no split beyond the longest shard
    *nsplit = static_cast<int32_t>(n);
    *split_len = len;
    if (n <= 1) {
        *scratch_bytes = 0;
    } else {
        const int64_t parts = static_cast<int64_t>(cp) * n * rows;  // (token, split, shard, head)
        *scratch_bytes = static_cast<size_t>(parts * kMlaVDim * 2 + parts * 4 * 2);  // rows, LSEs, scales
    }
}

VarlenLayout varlen_layout(int64_t B, int hq, int64_t T, int cp) {
    VarlenLayout l{};
    const int64_t rbt = (hq + kMlaRowsPerBlock - 1) / kMlaRowsPerBlock;
    l.pairs = B * rbt * cp;
    l.items = l.pairs + kVarlenTarget;
    // A pair splits only when it has more than kMlaMinSplitTiles tiles.
    const int64_t shard_tiles = ((T + cp - 1) / cp + kMlaKeysPerTile - 1) / kMlaKeysPerTile;
    const int64_t max_n = (shard_tiles + kMlaMinSplitTiles - 1) / kMlaMinSplitTiles;
    l.slots = max_n > 1 ? std::min<int64_t>(2 * kVarlenTarget, l.pairs * max_n) : 0;
    const size_t rows = static_cast<size_t>(l.slots) * kMlaRowsPerBlock;
    l.off_lse = rows * kMlaVDim * sizeof(uint16_t);
    l.off_scale = l.off_lse + rows * sizeof(float);
    l.off_hdr = (l.off_scale + rows * sizeof(float) + 63) / 64 * 64;
    l.off_items = l.off_hdr + 64;
    l.off_split = l.off_items + static_cast<size_t>(l.items) * sizeof(VarlenItem);
    l.bytes = l.off_split + static_cast<size_t>(kVarlenTarget) * sizeof(VarlenSplit);
    return l;
}

int plan_mla(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv, int64_t T, int64_t kv_st,
             const MlaVarlen* vl, int dtype, int cp, float softmax_scale, int lse_mode, void* o, int64_t o_sb,
             int64_t o_sh, float* lse, int64_t lse_sb, void* scratch, size_t scratch_bytes, MlaPlan* plan,
             const char* fn_name) {
    const char* fn = fn_name ? fn_name : (vl ? "dcp_mla_partial_decode_varlen" : "dcp_mla_partial_decode");
    if (B < 0 || hq < 1 || T < 0)
        return fail(DCP_ERR_INVALID_ARG, "%s: need B >= 0, hq >= 1, %s >= 0 (got %lld, %d, %lld)", fn,
                    vl ? "max_seq_len" : "kv_tokens", (long long)B, hq, (long long)T);
    if (vl && vl->kv_layout != DCP_KV_CONTIGUOUS && vl->kv_layout != DCP_KV_INTERLEAVED)
        return fail(DCP_ERR_INVALID_ARG, "%s: kv_layout %d is neither DCP_KV_CONTIGUOUS nor DCP_KV_INTERLEAVED", fn,
                    vl->kv_layout);
    if (cp < 1 || cp > DCP_MAX_CP)
        return fail(DCP_ERR_INVALID_ARG, "%s: cp = %d is outside [1, %d]", fn, cp, DCP_MAX_CP);
    if (lse_mode != DCP_LSE_BASE_E && lse_mode != DCP_LSE_BASE_2)
        return fail(DCP_ERR_INVALID_ARG, "%s: lse_mode %d is neither DCP_LSE_BASE_E nor DCP_LSE_BASE_2", fn,
                    lse_mode);
    if (dtype != DCP_DTYPE_BF16 && dtype != DCP_DTYPE_FP16)
        return fail(DCP_ERR_LAYOUT, "%s: dtype %d is neither DCP_DTYPE_BF16 nor DCP_DTYPE_FP16", fn, dtype);
    if (!(softmax_scale > 0.0f) || std::isinf(softmax_scale))
        return fail(DCP_ERR_INVALID_ARG, "%s: softmax_scale must be a positive finite number", fn);
    if (B * static_cast<int64_t>(hq) > (int64_t{1} << 30))
        return fail(DCP_ERR_INVALID_ARG, "%s: B * hq = %lld query rows exceeds 2^30", fn, (long long)(B * hq));
    if (B == 0) {
        *plan = MlaPlan{};
        return ok();
    }
    if (!q || !o || !lse || (T > 0 && !kv))
        return fail(DCP_ERR_INVALID_ARG, "%s: q, o_part, lse_part (and kv when there are keys) must be non-null", fn);
    if (vl && !vl->seq_lens) return fail(DCP_ERR_INVALID_ARG, "%s: seq_lens must be non-null when B > 0", fn);
    if (vl && T > kVarlenMaxLen)
        return fail(DCP_ERR_INVALID_ARG, "%s: max_seq_len = %lld exceeds %d", fn, (long long)T, kVarlenMaxLen);
    if (vl && !aligned(vl->seq_lens, 4)) return fail(DCP_ERR_ALIGN, "%s: seq_lens must be 4-byte aligned", fn);
    const int64_t kv_sb = vl ? vl->kv_sb : 0;
    if (q_sb < 0 || q_sh < 0 || kv_st < 0 || kv_sb < 0 || o_sb < 0 || o_sh < 0 || lse_sb < 0)
        return fail(DCP_ERR_LAYOUT, "%s: strides must be non-negative", fn);
    if (kv_sb % 8) return fail(DCP_ERR_ALIGN, "%s: kv_sb must be a multiple of 8 elements", fn);
    const int64_t H = static_cast<int64_t>(cp) * hq;
    if (!rows_disjoint(B, o_sb, H, o_sh, kMlaVDim))
        return fail(DCP_ERR_LAYOUT, "%s: o_part rows overlap (o_sb = %lld, o_sh = %lld)", fn, (long long)o_sb,
                    (long long)o_sh);
    if (!rows_disjoint(B, lse_sb, H, 1, 1))
        return fail(DCP_ERR_LAYOUT, "%s: lse_sb = %lld < cp*hq = %lld makes lse_part rows overlap", fn,
                    (long long)lse_sb, (long long)H);
    if (!aligned(q, 16) || !aligned(o, 16) || (kv && !aligned(kv, 16)))
        return fail(DCP_ERR_ALIGN, "%s: q, kv and o_part must be 16-byte aligned", fn);
    if (q_sb % 8 || q_sh % 8 || kv_st % 8 || o_sb % 8 || o_sh % 8)
        return fail(DCP_ERR_ALIGN, "%s: q_sb, q_sh, kv_st, o_sb and o_sh must be multiples of 8 elements", fn);
    if (!aligned(lse, 4)) return fail(DCP_ERR_ALIGN, "%s: lse_part must be 4-byte aligned", fn);
    // Offsets inside one key tile are 32-bit element counts; interleaved rows
    // of a tile are cp rows apart.
    const int64_t row_step = (vl && vl->kv_layout == DCP_KV_INTERLEAVED) ? cp : 1;
    if (kv_st * row_step > ((int64_t{1} << 31) - kMlaQkDim) / kMlaKeysPerTile)
        return fail(DCP_ERR_LAYOUT, "%s: kv_st = %lld is too large (at most %lld elements)", fn, (long long)kv_st,
                    (long long)(((int64_t{1} << 31) - kMlaQkDim) / kMlaKeysPerTile / row_step));

    int32_t nsplit = 1;
    int64_t split_len = 0;
    size_t need;
    VarlenLayout vlay{};
    if (vl) {
        vlay = varlen_layout(B, hq, T, cp);
        if (vlay.items >= (int64_t{1} << 31))
            return fail(DCP_ERR_INVALID_ARG, "%s: %lld work items exceed one launch (fewer tokens per call)", fn,
                        (long long)vlay.items);
        need = vlay.bytes;
    } else {
        mla_split(B, hq, T, cp, &nsplit, &split_len, &need);
    }
    if (need > 0 && (!scratch || scratch_bytes < need))
        return fail(DCP_ERR_WORKSPACE, "%s: needs %zu bytes of scratch (%s_scratch_size), got %zu", fn, need, fn,
                    scratch ? scratch_bytes : size_t{0});
    if (need > 0 && !aligned(scratch, 16)) return fail(DCP_ERR_ALIGN, "%s: scratch must be 16-byte aligned", fn);

    const Extent e_q = extent(q, B, q_sb, hq, q_sh, kMlaQkDim, 2);
    const Extent e_kv = T > 0 ? extent(kv, vl ? B : 1, kv_sb, T, kv_st, kMlaQkDim, 2) : Extent{0, 0};
    const Extent e_o = extent(o, B, o_sb, H, o_sh, kMlaVDim, 2);
    const Extent e_l = extent(lse, B, lse_sb, 1, 0, H, 4);
    if (overlaps(e_o, e_q) || overlaps(e_o, e_kv) || overlaps(e_l, e_q) || overlaps(e_l, e_kv) ||
        overlaps(e_l, e_o))
        return fail(DCP_ERR_INVALID_ARG, "%s: o_part / lse_part overlap an input or each other", fn);
    if (need > 0) {
        const Extent e_s{reinterpret_cast<uintptr_t>(scratch), reinterpret_cast<uintptr_t>(scratch) + need};
        if (overlaps(e_s, e_q) || overlaps(e_s, e_kv) || overlaps(e_s, e_o) || overlaps(e_s, e_l))
            return fail(DCP_ERR_INVALID_ARG, "%s: scratch overlaps an input or an output", fn);
    }

    MlaArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kv = static_cast<const uint16_t*>(kv);
    a.q_sb = q_sb;
    a.q_sh = q_sh;
    a.kv_st = kv_st;
    a.T = T;
    a.split_len = split_len;
    a.rows = static_cast<int32_t>(B * hq);
    a.hq = hq;
    a.cp = cp;
    a.nsplit = nsplit;
    a.row_blocks = (a.rows + kMlaRowsPerBlock - 1) / kMlaRowsPerBlock;
    a.dtype = dtype;
    if (vl) {
        a.seq_lens = vl->seq_lens;
        a.kv_sb = vl->kv_sb;
        a.interleaved = vl->kv_layout == DCP_KV_INTERLEAVED ? 1 : 0;
        a.rb_per_token = (hq + kMlaRowsPerBlock - 1) / kMlaRowsPerBlock;
        a.row_blocks = static_cast<int32_t>(B * a.rb_per_token);
        char* base = static_cast<char*>(scratch);
        a.part_o = reinterpret_cast<uint16_t*>(base);
        a.part_lse = reinterpret_cast<float*>(base + vlay.off_lse);
        a.part_scale = reinterpret_cast<float*>(base + vlay.off_scale);
        a.vl_hdr = reinterpret_cast<VarlenHeader*>(base + vlay.off_hdr);
        a.vl_items = reinterpret_cast<VarlenItem*>(base + vlay.off_items);
        a.vl_splits = reinterpret_cast<VarlenSplit*>(base + vlay.off_split);
        a.slots = vlay.slots;
    }
    a.scale_log2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
    a.lse_scale = lse_mode == DCP_LSE_BASE_2 ? 1.0f : 0.6931471805599453f;
    *plan = MlaPlan{};
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.o_sb = o_sb;
    a.o_sh = o_sh;
    a.lse_sb = lse_sb;
    if (!vl && nsplit > 1) {
        // Per-split scaled fp16 partials in the scratch buffer, then the merge over splits.
        const int64_t heads = static_cast<int64_t>(nsplit) * H;   // per token
        a.part_o = static_cast<uint16_t*>(scratch);
        a.part_lse = reinterpret_cast<float*>(a.part_o + B * heads * kMlaVDim);
        a.part_scale = a.part_lse + B * heads;
        a.part_sb = heads;
        MergeArgs m{};
        m.attn = a.part_o;
        m.in_dtype = kPayloadF16Scaled;
        m.lse = a.part_lse;
        m.sc_off = B * heads;          // part_scale sits right after part_lse
        m.out = static_cast<uint16_t*>(o);
        m.out_lse = lse;
        m.a_sb = heads * kMlaVDim;
        m.a_sj = kMlaVDim;             // local head j = s*hq + h
        m.a_ss = H * kMlaVDim;         // split p
        m.l_sb = heads;
        m.l_sj = 1;
        m.l_ss = H;
        m.o_sb = o_sb;
        m.o_sj = o_sh;
        m.ol_sb = lse_sb;
        m.h_local = static_cast<int32_t>(H);
        m.cp = nsplit;
        m.dtype = dtype;
        m.cached = 1;                  // the partials were written just before
        m.rows = 0;                    // set per token chunk at launch
        m.to_log2 = lse_mode == DCP_LSE_BASE_2 ? 1.0f : 1.4426950408889634f;
        m.from_log2 = lse_mode == DCP_LSE_BASE_2 ? 1.0f : 0.6931471805599453f;
        if (!merge_strides_fit(m))
            return fail(DCP_ERR_INVALID_ARG, "%s: %lld split partials per token are too many (fewer heads per call)",
                        fn, (long long)heads);
        plan->reduce = m;
    }
    plan->args = a;
    plan->scratch_bytes = need;
    plan->blocks = vl ? vlay.items : static_cast<int64_t>(a.row_blocks) * cp * nsplit;
    plan->varlen = vl != nullptr;
    // One row block: no other workgroup reads a key range, so every tile comes
    // from HBM; the decode keeps two tiles in flight instead of one.
    plan->deep = vl == nullptr && a.row_blocks == 1;
    if (plan->blocks >= (int64_t{1} << 31))
        return fail(DCP_ERR_INVALID_ARG, "%s: %lld workgroups exceed one launch (fewer tokens per call)", fn,
                    (long long)plan->blocks);
    plan->B = B;
    return ok();
}

namespace {
// The checks dcp_workspace_size and dcp_workspace_create share.
int check_geometry(const char* fn, int64_t capacity_tokens, int h_local, int cp, int d, int dtype) {
    if (capacity_tokens < 1)
        return fail(DCP_ERR_INVALID_ARG, "%s: capacity_tokens = %lld must be >= 1", fn, (long long)capacity_tokens);
    if (h_local < 1 || cp < 1 || cp > DCP_MAX_CP)
        return fail(DCP_ERR_INVALID_ARG, "%s: need h_local >= 1 and 1 <= cp <= %d (got %d, %d)", fn, DCP_MAX_CP,
                    h_local, cp);
    if (d != DCP_HEAD_DIM)
        return fail(DCP_ERR_LAYOUT, "%s: head dimension %d is not supported (only %d)", fn, d, DCP_HEAD_DIM);
    if (dtype != DCP_DTYPE_BF16 && dtype != DCP_DTYPE_FP16)
        return fail(DCP_ERR_LAYOUT, "%s: dtype %d is not supported (DCP_DTYPE_BF16 or DCP_DTYPE_FP16)", fn, dtype);
    // One launch covers capacity * h_local rows, counted in 32 bits.
    if (capacity_tokens * static_cast<int64_t>(h_local) > (int64_t{1} << 30))
        return fail(DCP_ERR_INVALID_ARG, "%s: capacity_tokens * h_local = %lld exceeds 2^30 rows per launch", fn,
                    (long long)(capacity_tokens * h_local));
    return DCP_OK;
}
}  // namespace

size_t merged_counter_bytes(int64_t B, int hq, int cp) {
    const int64_t row_blocks = (B * hq + kMlaRowsPerBlock - 1) / kMlaRowsPerBlock;
    return static_cast<size_t>((row_blocks * (cp + 1) * 4 + 255) / 256 * 256);
}

// dcp_mla_decode_merged: the producer's plan with the split partials placed
// after the arrival counters, plus the shard merge (fused into the decode
// kernel's epilogue, or as its own launches).
int plan_mla_merged(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv, int64_t T,
                    int64_t kv_st, int dtype, int cp, float softmax_scale, int lse_mode, void* o, int64_t o_sb,
                    int64_t o_sh, float* lse, int64_t lse_sb, void* out, int64_t out_sb, int64_t out_sh,
                    float* out_lse, int64_t out_lse_sb, int fuse, void* scratch, size_t scratch_bytes,
                    MlaPlan* plan) {
    const char* fn = "dcp_mla_decode_merged";
    if (fuse != DCP_FUSE_NONE && fuse != DCP_FUSE_EPILOGUE && fuse != DCP_FUSE_AUTO && fuse != DCP_FUSE_REDUCTIONS)
        return fail(DCP_ERR_INVALID_ARG,
                    "%s: fuse %d is not DCP_FUSE_NONE, DCP_FUSE_EPILOGUE, DCP_FUSE_REDUCTIONS or DCP_FUSE_AUTO", fn,
                    fuse);
    if (B < 0 || hq < 1 || T < 0 || cp < 1 || cp > DCP_MAX_CP || B * static_cast<int64_t>(hq) > (int64_t{1} << 30))
        return fail(DCP_ERR_INVALID_ARG, "%s: need B >= 0, hq >= 1, kv_tokens >= 0, 1 <= cp <= %d and B * hq <= 2^30",
                    fn, DCP_MAX_CP);
    const size_t cnt = merged_counter_bytes(B, hq, cp);
    int32_t nsplit;
    int64_t split_len;
    size_t part;
    mla_split(B, hq, T, cp, &nsplit, &split_len, &part);
    if (B > 0 && (!scratch || scratch_bytes < cnt + part))
        return fail(DCP_ERR_WORKSPACE, "%s: needs %zu bytes of zero-filled scratch (%s_scratch_size), got %zu", fn,
                    cnt + part, fn, scratch ? scratch_bytes : size_t{0});
    char* parts = scratch ? static_cast<char*>(scratch) + cnt : nullptr;
    const int rc = plan_mla(q, B, hq, q_sb, q_sh, kv, T, kv_st, nullptr, dtype, cp, softmax_scale, lse_mode, o, o_sb,
                            o_sh, lse, lse_sb, parts, scratch ? scratch_bytes - cnt : 0, plan, fn);
    if (rc != DCP_OK) return rc;
    plan->merge_shards = false;
    plan->reduce_merge = false;
    if (B == 0) return ok();
    if (!out) return fail(DCP_ERR_INVALID_ARG, "%s: out must be non-null when B > 0", fn);
    if (out_sb < 0 || out_sh < 0 || out_lse_sb < 0) return fail(DCP_ERR_LAYOUT, "%s: strides must be non-negative", fn);
    if (!rows_disjoint(B, out_sb, hq, out_sh, kMlaVDim))
        return fail(DCP_ERR_LAYOUT, "%s: out rows overlap (out_sb = %lld, out_sh = %lld)", fn, (long long)out_sb,
                    (long long)out_sh);
    if (out_lse && !rows_disjoint(B, out_lse_sb, hq, 1, 1))
        return fail(DCP_ERR_LAYOUT, "%s: out_lse_sb = %lld < hq = %d makes out_lse rows overlap", fn,
                    (long long)out_lse_sb, hq);
    if (!aligned(out, 16) || out_sb % 8 || out_sh % 8)
        return fail(DCP_ERR_ALIGN, "%s: out must be 16-byte aligned with out_sb, out_sh multiples of 8 elements", fn);
    if (out_lse && !aligned(out_lse, 4)) return fail(DCP_ERR_ALIGN, "%s: out_lse must be 4-byte aligned", fn);
    if (!aligned(scratch, 16)) return fail(DCP_ERR_ALIGN, "%s: scratch must be 16-byte aligned", fn);
    const int64_t H = static_cast<int64_t>(cp) * hq;
    const Extent e_q = extent(q, B, q_sb, hq, q_sh, kMlaQkDim, 2);
    const Extent e_kv = T > 0 ? extent(kv, 1, 0, T, kv_st, kMlaQkDim, 2) : Extent{0, 0};
    const Extent e_o = extent(o, B, o_sb, H, o_sh, kMlaVDim, 2);
    const Extent e_l = extent(lse, B, lse_sb, 1, 0, H, 4);
    const Extent e_s{reinterpret_cast<uintptr_t>(scratch), reinterpret_cast<uintptr_t>(scratch) + cnt + part};
    const Extent e_out = extent(out, B, out_sb, hq, out_sh, kMlaVDim, 2);
    if (overlaps(e_out, e_q) || overlaps(e_out, e_kv) || overlaps(e_out, e_o) || overlaps(e_out, e_l) ||
        overlaps(e_out, e_s))
        return fail(DCP_ERR_INVALID_ARG, "%s: out overlaps an input, o_part, lse_part or the scratch", fn);
    if (out_lse) {
        const Extent e_ol = extent(out_lse, B, out_lse_sb, 1, 0, hq, 4);
        if (overlaps(e_ol, e_q) || overlaps(e_ol, e_kv) || overlaps(e_ol, e_o) || overlaps(e_ol, e_l) ||
            overlaps(e_ol, e_s) || overlaps(e_ol, e_out))
            return fail(DCP_ERR_INVALID_ARG, "%s: out_lse overlaps another buffer", fn);
    }

    MlaArgs& a = plan->args;
    // DCP_FUSE_AUTO never takes the fused epilogue (measured slower at small
    // B, where the agent-scope publication of each workgroup's part costs more
    // than the launches it saves, and even from B = 32 on); with many key
    // splits and cp <= 16 it takes the combined reduction launch, else the
    // separate launches.
    a.fused = fuse == DCP_FUSE_EPILOGUE ? 1 : 0;
    a.split_cnt = static_cast<int32_t*>(scratch);
    a.rb_cnt = a.split_cnt + static_cast<int64_t>(a.row_blocks) * cp;
    a.out = static_cast<uint16_t*>(out);
    a.out_lse = out_lse;
    a.out_sb = out_sb;
    a.out_sh = out_sh;
    a.out_lse_sb = out_lse_sb;
    a.to_log2 = lse_mode == DCP_LSE_BASE_2 ? 1.0f : 1.4426950408889634f;
    a.from_log2 = lse_mode == DCP_LSE_BASE_2 ? 1.0f : 0.6931471805599453f;
    if (!a.fused) {
        // The shard merge as dcp_lse_combine runs it over (o, lse) in the
        // FlashMLA layout, the partials read with plain loads (just written).
        MergeArgs m{};
        m.attn = o;
        m.in_dtype = dtype;
        m.lse = lse;
        m.out = static_cast<uint16_t*>(out);
        m.out_lse = out_lse;
        m.a_sb = o_sb;
        m.a_sj = o_sh;
        m.a_ss = static_cast<int64_t>(hq) * o_sh;
        m.l_sb = lse_sb;
        m.l_sj = 1;
        m.l_ss = hq;
        m.o_sb = out_sb;
        m.o_sj = out_sh;
        m.ol_sb = out_lse_sb;
        m.h_local = hq;
        m.cp = cp;
        m.dtype = dtype;
        m.cached = 1;
        m.to_log2 = a.to_log2;
        m.from_log2 = a.from_log2;
        if (!merge_strides_fit(m))
            return fail(DCP_ERR_LAYOUT, "%s: o_part / lse_part strides must be below 2^31 elements", fn);
        plan->merge_shards = true;
        plan->shard_merge = m;
        // The combined launch needs the split reduction (several splits)
        // and at most 16 shards (one block holds every shard of a head).
        // AUTO takes it from 16 splits per shard on: measured (128 heads,
        // 4 shards) 1% faster at 64 and 32 splits, even at 8, 0.2% slower at 2.
        const bool can = a.nsplit > 1 && cp <= 16;
        plan->reduce_merge = can && (fuse == DCP_FUSE_REDUCTIONS || (fuse == DCP_FUSE_AUTO && a.nsplit >= 16));
    }
    return ok();
}

}  // namespace dcp

extern "C" {

int dcp_mla_decode_merged_scratch_size(int64_t B, int hq, int64_t kv_tokens, int cp, size_t* bytes) {
    if (!bytes) return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_decode_merged_scratch_size: bytes is null");
    if (B < 0 || hq < 1 || kv_tokens < 0 || cp < 1 || cp > DCP_MAX_CP || B * static_cast<int64_t>(hq) > (int64_t{1} << 30))
        return dcp::fail(DCP_ERR_INVALID_ARG,
                         "dcp_mla_decode_merged_scratch_size: need B >= 0, hq >= 1, kv_tokens >= 0, 1 <= cp <= %d, "
                         "B * hq <= 2^30",
                         DCP_MAX_CP);
    int32_t n;
    int64_t len;
    size_t part;
    dcp::mla_split(B, hq, kv_tokens, cp, &n, &len, &part);
    *bytes = B == 0 ? 0 : dcp::merged_counter_bytes(B, hq, cp) + part;
    return dcp::ok();
}

int dcp_mla_partial_decode_scratch_size(int64_t B, int hq, int64_t kv_tokens, int cp, size_t* bytes) {
    if (!bytes) return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_partial_decode_scratch_size: bytes is null");
    if (B < 0 || hq < 1 || kv_tokens < 0 || cp < 1 || cp > DCP_MAX_CP)
        return dcp::fail(DCP_ERR_INVALID_ARG,
                         "dcp_mla_partial_decode_scratch_size: need B >= 0, hq >= 1, kv_tokens >= 0, 1 <= cp <= %d",
                         DCP_MAX_CP);
    if (B * static_cast<int64_t>(hq) > (int64_t{1} << 30))
        return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_partial_decode_scratch_size: B * hq exceeds 2^30");
    int32_t n;
    int64_t len;
    dcp::mla_split(B, hq, kv_tokens, cp, &n, &len, bytes);
    return dcp::ok();
}

int dcp_mla_partial_decode_varlen_scratch_size(int64_t B, int hq, int64_t max_seq_len, int cp, size_t* bytes) {
    if (!bytes) return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_partial_decode_varlen_scratch_size: bytes is null");
    if (B < 0 || hq < 1 || max_seq_len < 0 || cp < 1 || cp > DCP_MAX_CP)
        return dcp::fail(DCP_ERR_INVALID_ARG,
                         "dcp_mla_partial_decode_varlen_scratch_size: need B >= 0, hq >= 1, max_seq_len >= 0, "
                         "1 <= cp <= %d",
                         DCP_MAX_CP);
    if (B * static_cast<int64_t>(hq) > (int64_t{1} << 30))
        return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_partial_decode_varlen_scratch_size: B * hq exceeds 2^30");
    if (max_seq_len > dcp::kVarlenMaxLen)
        return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_mla_partial_decode_varlen_scratch_size: max_seq_len = %lld exceeds %d",
                         (long long)max_seq_len, dcp::kVarlenMaxLen);
    *bytes = B == 0 ? 0 : dcp::varlen_layout(B, hq, max_seq_len, cp).bytes;
    return dcp::ok();
}


int dcp_workspace_size(int64_t capacity_tokens, int h_local, int cp, int d, int dtype, size_t* bytes) {
    if (!bytes) return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_workspace_size: bytes (the output) is null");
    const int rc = dcp::check_geometry("dcp_workspace_size", capacity_tokens, h_local, cp, d, dtype);
    if (rc != DCP_OK) return rc;
    *bytes = dcp::workspace_layout(capacity_tokens, h_local, cp, d).bytes;
    return dcp::ok();
}

int dcp_workspace_create(void* dev_buf, size_t bytes, int64_t capacity_tokens, int h_local, int cp, int d, int dtype,
                         void* hip_stream, dcp_workspace** ws) {
    const char* fn = "dcp_workspace_create";
    if (!ws) return dcp::fail(DCP_ERR_INVALID_ARG, "%s: ws (the output handle) is null", fn);
    *ws = nullptr;
    const int rc = dcp::check_geometry(fn, capacity_tokens, h_local, cp, d, dtype);
    if (rc != DCP_OK) return rc;
    const size_t need = dcp::workspace_layout(capacity_tokens, h_local, cp, d).bytes;
    if (!dev_buf || bytes < need)
        return dcp::fail(DCP_ERR_WORKSPACE,
                         "%s: the device buffer must hold %zu bytes for capacity %lld x %d local heads x %d shards "
                         "(dcp_workspace_size); got %zu bytes at %p",
                         fn, need, (long long)capacity_tokens, h_local, cp, dev_buf ? bytes : size_t{0}, dev_buf);
    if (reinterpret_cast<uintptr_t>(dev_buf) % 16)
        return dcp::fail(DCP_ERR_ALIGN, "%s: the device buffer (%p) must be 16-byte aligned", fn, dev_buf);
    dcp_workspace* w = new (std::nothrow) dcp_workspace;
    if (!w) return dcp::fail(DCP_ERR_INVALID_ARG, "%s: out of host memory", fn);
    w->capacity = capacity_tokens;
    w->h_local = h_local;
    w->cp = cp;
    w->d = d;
    w->dtype = dtype;
    w->load_policy = DCP_LOAD_STREAMING;
    w->stream = hip_stream;
    w->buf = dev_buf;
    w->bytes = bytes;
    w->magic = dcp::kWorkspaceMagic;
    *ws = w;
    return dcp::ok();
}

int dcp_workspace_recv(const dcp_workspace* ws, void** attn, int64_t* attn_sb, int64_t* attn_sh, float** lse,
                       int64_t* lse_sb) {
    if (!ws || ws->magic != dcp::kWorkspaceMagic)
        return dcp::fail(DCP_ERR_WORKSPACE, "dcp_workspace_recv: not a workspace (or destroyed)");
    if (!attn || !attn_sb || !attn_sh || !lse || !lse_sb)
        return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_workspace_recv: every output pointer must be non-null");
    const int64_t H = static_cast<int64_t>(ws->cp) * ws->h_local;
    const dcp::WorkspaceLayout l = dcp::workspace_layout(ws->capacity, ws->h_local, ws->cp, ws->d);
    *attn = ws->buf;
    *attn_sh = ws->d;
    *attn_sb = H * ws->d;
    *lse = reinterpret_cast<float*>(static_cast<char*>(ws->buf) + l.lse_off);
    *lse_sb = H;
    return dcp::ok();
}

int dcp_workspace_destroy(dcp_workspace* ws) {
    if (!ws) return dcp::ok();
    if (ws->magic != dcp::kWorkspaceMagic)
        return dcp::fail(DCP_ERR_WORKSPACE, "dcp_workspace_destroy: not a workspace (or destroyed twice)");
    ws->magic = 0;
    delete ws;
    return dcp::ok();
}

int dcp_workspace_set_load_policy(dcp_workspace* ws, int policy) {
    if (!ws || ws->magic != dcp::kWorkspaceMagic)
        return dcp::fail(DCP_ERR_INVALID_ARG, "dcp_workspace_set_load_policy: not a workspace");
    if (policy != DCP_LOAD_STREAMING && policy != DCP_LOAD_CACHED)
        return dcp::fail(DCP_ERR_INVALID_ARG,
                         "dcp_workspace_set_load_policy: policy %d is neither DCP_LOAD_STREAMING nor DCP_LOAD_CACHED",
                         policy);
    ws->load_policy = policy;
    return dcp::ok();
}

const char* dcp_last_error(void) { return dcp::g_error; }

const char* dcp_status_string(int status) {
    switch (status) {
        case DCP_OK: return "DCP_OK";
        case DCP_ERR_INVALID_ARG: return "DCP_ERR_INVALID_ARG";
        case DCP_ERR_LAYOUT: return "DCP_ERR_LAYOUT";
        case DCP_ERR_ALIGN: return "DCP_ERR_ALIGN";
        case DCP_ERR_STREAM: return "DCP_ERR_STREAM";
        case DCP_ERR_WORKSPACE: return "DCP_ERR_WORKSPACE";
        case DCP_ERR_HIP: return "DCP_ERR_HIP";
        default: return "DCP_ERR_UNKNOWN";
    }
}

}  // extern "C"
