// dcp_internal.h -- host-side types shared by the validator (dcp_host.cpp) and
// the HIP launch code (merge.hip).  No HIP types appear here, so the validator
// builds with a plain host compiler too.
#pragma once

#include <cstddef>
#include <cstdint>

#include "dcp.h"

namespace dcp {

// Kernel parameters of one merge launch, after the layout adapter has turned
// the caller's [B, H, D] attention buffer and its LSE layout into one strided
// (token b, local head j, shard s) addressing scheme:
//   O(b, j, s, :)  at attn    + b*a_sb + j*a_sj + s*a_ss      (elements of in_dtype)
//   lse(b, j, s)   at lse     + b*l_sb + j*l_sj + s*l_ss      (fp32 elements)
//   out(b, j, :)   at out     + b*o_sb + j*o_sj               (bf16 elements)
//   L(b, j)        at out_lse + b*ol_sb + j                   (fp32, optional)
// Rows are r = b*h_local + j, r < rows.
struct MergeArgs {
    const void* attn;
    const float* lse;
    uint16_t* out;
    float* out_lse;
    int64_t a_sb, a_sj, a_ss;
    int64_t l_sb, l_sj, l_ss;
    int64_t o_sb, o_sj;
    int64_t ol_sb;
    int32_t rows;
    int32_t h_local;
    int32_t cp;
    int32_t in_dtype;   // attn: DCP_DTYPE_BF16, DCP_DTYPE_FP16 or kPayloadF16Scaled (internal)
    int32_t dtype;      // out: DCP_DTYPE_BF16 or DCP_DTYPE_FP16
    int32_t cached;     // 1: plain loads and stores; 0: non-temporal
    // (lse_s - M) * to_log2 is the exponent of 2 of the weight; log2(S) * from_log2
    // is added to M for the merged LSE.  Base 2: both 1.  Base e: log2 e and ln 2.
    float to_log2;
    float from_log2;
    // kPayloadF16Scaled: shard s of a row is scaled by the float sc_off
    // elements after its LSE (lse + b*l_sb + j*l_sj + s*l_ss + sc_off).
    int64_t sc_off;
};

// Most tokens one merge launch covers (the grid's second dimension).
constexpr int64_t kMaxLaunchTokens = 65535;

// Payload type of the merge input used only inside the library: the MLA
// decode's split partials, each row stored in fp16 after multiplication by
// an exact power of two (chosen so that the row's largest magnitude lies in
// [2^14, 2^15)), with the inverse factor stored beside the row's LSE.  The
// merge multiplies a split's normalised weight by that factor.  Never
// accepted from callers.
constexpr int32_t kPayloadF16Scaled = 100;

// Bytes of one payload element of a merge input type (every type is 16-bit).
inline int64_t payload_bytes(int32_t) { return 2; }

// The arguments `a` moved to start at token t0 and cover `tokens` tokens.
MergeArgs merge_args_at(const MergeArgs& a, int64_t t0, int64_t tokens);

// A validated merge call: the arguments of the first chunk plus how to step
// to the next one.
struct MergePlan {
    MergeArgs args;       // chunk 0; rows = tokens_in_chunk * h_local
    int64_t B;            // total tokens
    int64_t chunk;        // tokens per launch (capacity)
    int64_t n_chunks;     // ceil(B / chunk), 0 when B == 0
};

}  // namespace dcp

struct dcp_workspace {
    int64_t capacity;
    int h_local;
    int cp;
    int d;
    int dtype;
    int load_policy;  // DCP_LOAD_STREAMING or DCP_LOAD_CACHED
    void* stream;
    void* buf;        // the caller's device buffer: the landing zone
    size_t bytes;
    uint64_t magic;
};

namespace dcp {

constexpr uint64_t kWorkspaceMagic = 0x64637077736b7632ull;  // "dcpwskv2"

// The workspace's device buffer: the receive-buffer landing zone of up to
// `capacity` tokens, laid out as the [B, H, D] attention output that
// dcp_lse_combine reads (H = cp * h_local, head s*h_local + j holding shard
// s of local head j, rows of D elements back to back), then the LSEs in the
// FlashMLA [B, H] layout, each region starting on a 256-byte boundary.
struct WorkspaceLayout {
    size_t lse_off;  // bytes from the buffer's start to the LSE region
    size_t bytes;    // total
};
inline WorkspaceLayout workspace_layout(int64_t capacity, int h_local, int cp, int d) {
    const size_t rows = static_cast<size_t>(capacity) * static_cast<size_t>(h_local) * static_cast<size_t>(cp);
    const size_t payload = rows * static_cast<size_t>(d) * 2;
    WorkspaceLayout l;
    l.lse_off = (payload + 255) / 256 * 256;
    l.bytes = l.lse_off + (rows * 4 + 255) / 256 * 256;
    return l;
}

// Record a message for dcp_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

// Validate every argument of dcp_lse_combine and build its launch plan.
// Touches no device memory and calls no HIP function.
int plan_merge(const dcp_workspace* ws, const void* attn, int64_t B, int H, int64_t attn_sb, int64_t attn_sh,
               const float* lse, int lse_layout, int64_t l0, int64_t l1, int64_t l2, int lse_mode, void* out,
               int64_t out_sb, int64_t out_sh, float* out_lse, int64_t out_lse_sb, void* hip_stream,
               MergePlan* plan);

// Arguments of chunk k of a plan (token range [k*chunk, min((k+1)*chunk, B))).
MergeArgs chunk_args(const MergePlan& plan, int64_t k);

// The merge kernels take the payload and LSE strides as 32-bit values (so
// that they fit the SGPRs the hardware preloads): true when every one of
// them is below 2^31 in magnitude.
inline bool merge_strides_fit(const MergeArgs& a) {
    const int64_t lim = int64_t{1} << 31;
    const int64_t v[6] = {a.a_sb, a.a_sj, a.a_ss, a.l_sb, a.l_sj, a.l_ss};
    for (int64_t x : v)
        if (x >= lim || x <= -lim) return false;
    return true;
}

// Enqueue one merge launch of already validated arguments (rows = tokens *
// h_local with at most kMaxLaunchTokens tokens) on `stream` (a hipStream_t).
// Returns the HIP error code of the launch (0 = success).
int merge_launch(const MergeArgs& a, void* stream);

// ---------------------------------------------------------------- MLA decode

constexpr int kMlaQkDim = DCP_QK_DIM;   // 576 query/key columns
constexpr int kMlaVDim = DCP_HEAD_DIM;  // 512 value columns
constexpr int kMlaRowsPerBlock = 128;   // query rows per workgroup
constexpr int kMlaKeysPerTile = 32;     // keys per LDS tile
constexpr int kMlaTargetBlocks = 256;   // split the KV until about this many workgroups (one per CU)
constexpr int kMlaMinSplitKeys = 256;   // ... but never below this many keys per split
constexpr int kMlaMaxSplits = DCP_MAX_CP;  // ... nor above what the merge kernel reduces in one launch

// Kernel parameters of the MLA split-KV decode.  Query row r = b*hq + h.
// The keys of shard s are [floor(s*T/cp), floor((s+1)*T/cp)); split p of a
// shard covers its keys [p*split_len, (p+1)*split_len).
// With one split the kernel writes the output of (b, shard s, head h) in the
// element type to o + b*o_sb + (s*hq + h)*o_sh and its LSE to
// lse + b*lse_sb + s*hq + h.  With several, split p writes its normalised
// output (kPayloadF16Scaled), LSE and scale as head u = p*cp*hq + s*hq + h of
// the scratch buffer: part_o [B][nsplit*cp*hq][512] fp16, then part_lse and
// part_scale [B][nsplit*cp*hq] fp32, which the merge kernel then reduces over
// p (an LSE merge with nsplit shards and cp*hq local heads) into o / lse.
// ------------------------------------------- variable-length work plan
// With per-token lengths the split length cannot be fixed on the host: a
// one-workgroup planning kernel reads seq_lens, picks a split length (in key
// tiles) so that the whole batch makes about kVarlenTarget splits, never
// fewer than kMlaMinSplitTiles tiles long, and writes the work list -- one
// item per split of every pair (token, row block, shard), longest first --
// into the scratch buffer.  Workgroup i of the decode kernel runs item i.  A
// pair with one split writes its output directly; a pair with n > 1 splits
// writes n scaled fp16 partials to consecutive slots (kMlaRowsPerBlock rows
// of 512 each, with an LSE and a scale per row), which a reduction kernel
// merges.  Pair index
// q = (b * rb_per_token + row block) * cp + s.
constexpr int kVarlenTarget = 256;       // splits over the whole batch (about one per compute unit)
constexpr int kMlaMinSplitTiles = kMlaMinSplitKeys / kMlaKeysPerTile;  // shortest split
constexpr int kMlaPlanThreads = 1024;  // the planning workgroup; also its number of size bins

struct VarlenHeader {
    int32_t n_items;      // items in the list; workgroups past it exit
    int32_t n_split;      // pairs with more than one split
    int64_t split_tiles;  // key tiles per split (at most kVarlenMaxLen)
};
struct VarlenItem {
    int32_t pair, p;      // split p of pair q
    int32_t slot;         // partial slot, or -1: the pair has one split
    int32_t pad;
};
struct VarlenSplit {
    int32_t pair, first, n, pad;  // the pair's partials are slots first .. first + n - 1
};

// The plan's arithmetic, shared by the kernels and the host-side checks.
#if defined(__HIP__)
#define DCP_HD __host__ __device__
#else
#define DCP_HD
#endif

// Token lengths are at most kVarlenMaxLen (checked on the host), so the
// per-pair arithmetic below is exact in 32 bits: the GPU has no integer
// divide, and a 64-bit division costs several times a 32-bit one.
constexpr int32_t kVarlenMaxLen = int32_t{1} << 30;

// Key tiles of shard s of a token with L rows (contiguous slices
// [floor(s L / cp), floor((s+1) L / cp)) or every cp-th row from row s).
// With L = q cp + r, floor(k L / cp) = k q + floor(k r / cp).
DCP_HD inline int32_t varlen_shard_tiles(int32_t L, int32_t s, int32_t cp, bool interleaved) {
    int32_t n;
    if (interleaved) {
        n = L > s ? (L - s + cp - 1) / cp : 0;
    } else {
        const int32_t q = L / cp, r = L - q * cp;
        n = q + ((s + 1) * r) / cp - (s * r) / cp;
    }
    return (n + kMlaKeysPerTile - 1) / kMlaKeysPerTile;
}
// Tiles per split for a batch of `total` tiles.  Capped at kVarlenMaxLen: a
// split that long already holds any shard whole (no pair splits).
DCP_HD inline int32_t varlen_split_tiles(int64_t total) {
    int64_t st = (total + kVarlenTarget - 1) / kVarlenTarget;
    if (st < kMlaMinSplitTiles) st = kMlaMinSplitTiles;
    return st > kVarlenMaxLen ? kVarlenMaxLen : static_cast<int32_t>(st);
}
// Splits of a pair of t tiles (an empty pair still has one, to write 0 / -inf).
DCP_HD inline int32_t varlen_splits(int32_t t, int32_t st) { return t > st ? (t + st - 1) / st : 1; }
// Size bin of a split of `size` <= st tiles: 0 (empty) .. kMlaPlanThreads - 1
// (full), rounded from size / st in fp32 (the bins only order the work list;
// both passes of the plan compute them identically).
DCP_HD inline int varlen_bin(int32_t size, int32_t st) {
    const float x = static_cast<float>(size) * static_cast<float>(kMlaPlanThreads - 1) / static_cast<float>(st);
    const int b = static_cast<int>(x + 0.5f);
    return b < kMlaPlanThreads - 1 ? b : kMlaPlanThreads - 1;
}

// Scratch layout of the variable-length producer: part_o [slots][128][512]
// fp16 (kPayloadF16Scaled), part_lse and part_scale [slots][128] fp32, the
// header, the items, the split list.
// With st >= total / target tiles per split the list holds at most
// pairs + target items, fewer than target split pairs and fewer than
// 2 * target partial slots (each split pair has more than st tiles).
struct VarlenLayout {
    int64_t pairs, items, slots;
    size_t off_lse, off_scale, off_hdr, off_items, off_split, bytes;
};
VarlenLayout varlen_layout(int64_t B, int hq, int64_t T, int cp);

struct MlaArgs {
    const uint16_t* q;      // row r at q + b*q_sb + h*q_sh, 576 columns
    const uint16_t* kv;     // token t at kv + t*kv_st, 576 columns
    uint16_t* o;
    float* lse;
    uint16_t* part_o;       // nsplit > 1: kPayloadF16Scaled rows
    float* part_lse;
    float* part_scale;      // the factor that undoes a partial row's scaling
    int64_t q_sb, q_sh, kv_st, o_sb, o_sh, lse_sb;
    int64_t part_sb;        // nsplit*cp*hq
    // Variable length (seq_lens != nullptr): token b attends over its own cache
    // kv + b*kv_sb, rows t < min(max(seq_lens[b], 0), T); a workgroup's rows
    // never span tokens (rb_per_token blocks of up to 128 heads per token).
    const int32_t* seq_lens;
    int64_t kv_sb;
    int32_t interleaved;    // shard s owns rows t with t mod cp == s (else a contiguous slice)
    int32_t rb_per_token;
    int64_t T;
    int64_t split_len;      // multiple of kMlaKeysPerTile
    int32_t rows;           // B * hq
    int32_t hq;
    int32_t cp;
    int32_t nsplit;
    int32_t row_blocks;     // ceil(rows / kMlaRowsPerBlock)
    int32_t dtype;          // DCP_DTYPE_BF16 or DCP_DTYPE_FP16 (q, kv, o)
    float scale_log2;       // softmax_scale * log2 e
    float lse_scale;        // lse = log2-domain LSE * lse_scale (1 for base 2, ln 2 for base e)
    // Variable length: the work list (part_o / part_lse are then the slots).
    VarlenHeader* vl_hdr;
    VarlenItem* vl_items;
    VarlenSplit* vl_splits;
    int64_t slots;          // partial slots in the scratch (0: no pair may split)
    // Fused epilogue (fixed length only): arrival counters (zero between
    // calls) and the merged output.  The last workgroup of (row block rb,
    // shard s) to count itself into split_cnt[rb*cp + s] reduces the shard's
    // splits into o / lse; the last shard of rb to count itself into
    // rb_cnt[rb] merges the cp shards of its rows into out / out_lse.
    int32_t fused;
    int32_t* split_cnt;
    int32_t* rb_cnt;
    uint16_t* out;
    float* out_lse;
    int64_t out_sb, out_sh, out_lse_sb;
    float to_log2, from_log2;  // the merges' base constants (as in MergeArgs)
};

struct MlaPlan {
    MlaArgs args;
    size_t scratch_bytes;   // needed scratch (0 when nsplit == 1)
    int64_t blocks;         // workgroups of the main kernel (0: nothing to do)
    bool varlen;            // planning kernel, decode over the work list, split reduction
    bool deep;              // the decode loop with two tiles in flight (one row block)
    MergeArgs reduce;       // nsplit > 1: the merge over splits (all B tokens; launched in token chunks)
    int64_t B;
    // dcp_mla_decode_merged without the fused epilogue: the shard merge of
    // o / lse into out / out_lse (all B tokens; launched in token chunks).
    bool merge_shards;
    MergeArgs shard_merge;
    // DCP_FUSE_REDUCTIONS (nsplit > 1, cp <= 16): the split reduction and the
    // shard merge in one launch (reduce_merge_launch) instead of two.
    bool reduce_merge;
};

// Launch a merge over all B tokens of `m` in chunks of at most
// kMaxLaunchTokens tokens and 2^30 rows; returns the first HIP error.
int merge_launch_all(const MergeArgs& m, int64_t B, void* stream);
// The split reduction `r` and the shard merge `m` of dcp_mla_decode_merged in
// one launch per token chunk (merge.hip); m.cp <= 16.
int reduce_merge_launch(const MergeArgs& r, const MergeArgs& m, int64_t B, int hq, void* stream);

// Scratch of dcp_mla_decode_merged: the arrival counters (row_blocks * (cp + 1)
// int32, rounded to 256 bytes), then the split partials as for
// dcp_mla_partial_decode.
size_t merged_counter_bytes(int64_t B, int hq, int cp);

// Validate every argument of dcp_mla_decode_merged and build the plan.
int plan_mla_merged(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv, int64_t T,
                    int64_t kv_st, int dtype, int cp, float softmax_scale, int lse_mode, void* o, int64_t o_sb,
                    int64_t o_sh, float* lse, int64_t lse_sb, void* out, int64_t out_sb, int64_t out_sh,
                    float* out_lse, int64_t out_lse_sb, int fuse, void* scratch, size_t scratch_bytes,
                    MlaPlan* plan);

// The variable-length producer's planning kernel and split reduction,
// enqueued on `stream` (a hipStream_t); return the HIP error of the launch.
int varlen_plan_launch(const MlaArgs& a, void* stream);
int varlen_reduce_launch(const MlaArgs& a, void* stream);

// Split decision and scratch size of the fixed-length producer; pure
// arithmetic on the shape.
void mla_split(int64_t B, int hq, int64_t T, int cp, int32_t* nsplit, int64_t* split_len, size_t* scratch_bytes);

// The variable-length arguments of dcp_mla_partial_decode_varlen.
struct MlaVarlen {
    const int32_t* seq_lens;  // device, [B]
    int64_t kv_sb;            // elements between consecutive tokens' caches (0: one shared cache)
    int kv_layout;            // DCP_KV_CONTIGUOUS or DCP_KV_INTERLEAVED
};

// Validate every argument of dcp_mla_partial_decode (vl == nullptr: one cache
// of T rows shared by every token) or of dcp_mla_partial_decode_varlen (T is
// then max_seq_len) and build the plan.
int plan_mla(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv, int64_t T, int64_t kv_st,
             const MlaVarlen* vl, int dtype, int cp, float softmax_scale, int lse_mode, void* o, int64_t o_sb,
             int64_t o_sh, float* lse, int64_t lse_sb, void* scratch, size_t scratch_bytes, MlaPlan* plan,
             const char* fn_name = nullptr);

// Enqueue a validated plan on `stream` (a hipStream_t): the planning kernel
// (variable length), the decode kernel and the split reduction.  Returns a
// DCP status; `fn` names the entry point in error messages.
int run_mla(const MlaPlan& plan, void* stream, const char* fn);

}  // namespace dcp
