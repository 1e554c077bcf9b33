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
//   O(b, j, s, :)  at attn    + b*a_sb + j*a_sj + s*a_ss      (bf16 elements)
//   lse(b, j, s)   at lse     + b*l_sb + j*l_sj + s*l_ss      (fp32 elements)
//   out(b, j, :)   at out     + b*o_sb + j*o_sj               (bf16 elements)
//   L(b, j)        at out_lse + b*ol_sb + j                   (fp32, optional)
// Rows are r = b*h_local + j, r < rows.
struct MergeArgs {
    const uint16_t* attn;
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
    // (lse_s - M) * to_log2 is the exponent of 2 of the weight; log2(S) * from_log2
    // is added to M for the merged LSE.  Base 2: both 1.  Base e: log2 e and ln 2.
    float to_log2;
    float from_log2;
};

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
    void* stream;
    uint64_t magic;
};

namespace dcp {

constexpr uint64_t kWorkspaceMagic = 0x64637077736b7631ull;  // "dcpwskv1"

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

}  // namespace dcp
