// merge.hip -- the DCP LSE merge on gfx950 (MI355X) and the dcp_lse_combine
// entry point.
//
// What it computes: for every token b and local head j, the LSE-weighted merge
// of the cp shard partials of that head ("[DCP] Run fi_a2a on FlashInfer's
// fused all-to-all + LSE reduce", sglang PR #40539, Motivation/Modifications;
// "[Attention] Add direct symmetric-memory DCP A2A", vLLM PR #48897: weights
// formed in fp32, empty shards publish -inf and their payload is skipped):
//     M = max_s lse_s, w_s = 2^((lse_s - M) * c), S = sum_s w_s,
//     out = sum_s (w_s / S) O_s, L = M + log2(S) / c,
// with c = 1 for base-2 LSEs and c = log2 e for natural-log LSEs.
//
// Mapping to CDNA4.  The work is a pure stream: every partial is read once and
// every output written once, so the kernel is bound by HBM bandwidth, not by
// arithmetic, and is built to keep as many bytes in flight as possible:
//  * one 64-lane wavefront per (b, j) row; lane l owns columns [8l, 8l + 8) of
//    D = 512, so one 16-byte load per lane fetches a shard's whole 1 KiB
//    D-vector, fully coalesced;
//  * all of a row's shard loads are issued before any arithmetic waits on
//    them, together with the LSE loads, so a wave has cp KiB in flight and a
//    launch needs a single memory round trip;
//  * cp <= 16: the row's LSEs have a wave-uniform address and are read with
//    scalar loads, so max, exponentials and sum are formed once per wavefront
//    with no cross-lane step; a row whose weights are all nonzero takes a
//    plain FMA path, a row with an empty shard (weight exactly 0, which covers
//    lse = -inf) zeroes that shard's payload first, so it is never used;
//  * cp > 16: two or four wavefronts per row, each with 16 shards' loads in
//    flight; lane s holds lse_s, the maximum and the sum are DPP reductions
//    over the lanes (the sum in the one fixed tree every path uses for more
//    than 16 parts), each wavefront sums its 16 shards (one accumulation
//    group of the shared arithmetic) and one adds the groups' sums from LDS
//    in ascending order (the split partials of the MLA decode, many rows with
//    adjacent parts, take one wavefront per row instead, with the same
//    arithmetic);
//  * fp32 FMAs in ascending shard order (for cp > 16 within each group of
//    16), then the hardware round-to-nearest-
//    even convert to the payload type and one 16-byte store per lane.  The
//    payload is bf16 or fp16 (both are the pages' payload types); one kernel
//    instance per type, differing only in the widening and narrowing.  A
//    third instance, inside the library only, reduces the MLA decode's split
//    partials: fp16 rows stored multiplied by a power of two, whose inverse
//    factor (read beside the LSE) multiplies the split's normalised weight.
// The per-element arithmetic does not depend on B, on the chunking or on the
// grid, so chunked and unchunked calls give identical bits; it is the one in
// merge_row.h, which every merge of partials in the library uses.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dcp_internal.h"
#include "merge_row.h"

namespace dcp {
namespace {

using mrow::Bf16;
using mrow::F16;
using mrow::Payload16;
using mrow::u32x4;

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

// Grid: x = group g of kWavesPerBlock local heads, y = token b of the chunk;
// wavefront w of block (g, b) merges local head j = g * kWavesPerBlock + w.
// Blocks are dispatched x first, so consecutive blocks read consecutive head
// groups of one token: the chip streams one contiguous token slab after
// another rather than hopping between tokens.
// No integer division, and no branch anywhere between the loads and the
// store, so the compiler keeps every load of the row ahead of the first wait.
// When h_local is not a multiple of kWavesPerBlock the spare wavefronts of
// the last group take j = h_local - 1: they read what that row's wavefront
// reads and store the very same bits to the same place.
struct Row {
    int b, j;
};

__device__ __forceinline__ Row row_of(int h_local) {
    Row r;
    r.b = blockIdx.y;
    const int j = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
    r.j = j < h_local ? j : h_local - 1;
    return r;
}

// Kernel arguments.  What the first loads need leads the parameter list as
// scalars -- the payload and LSE pointers, their 32-bit element strides and
// h_local -- so that the hardware preloads them into SGPRs before the
// wavefront starts (gfx950 kernel-argument preloading, switched on by the
// build): the addresses are formed and the loads issued without first
// waiting on a scalar load of the argument block, one memory latency less per
// launch.  The rest is needed only once the loads are in flight and comes in
// one struct, read with ordinary scalar loads meanwhile.
struct MergeTail {
    uint16_t* out;
    float* out_lse;
    int64_t o_sb, o_sj, ol_sb;
    int64_t sc_off;  // scaled payloads: the factors, in floats after the LSEs
    float to_log2, from_log2;
    int32_t cp;
};

MergeTail tail_of(const MergeArgs& a) {
    return MergeTail{a.out, a.out_lse, a.o_sb, a.o_sj, a.ol_sb, a.sc_off, a.to_log2, a.from_log2, a.cp};
}

// The output row always leaves with a non-temporal store, under either load
// policy: measured, that is the faster store both when the partials stream in
// from HBM and when they are read from the caches (B = 512 hot: 5.05 us
// against 5.79 us with plain stores).
template <typename T>
__device__ __forceinline__ void store_row(const MergeTail& t, Row r, int lane, const float (&acc)[8], float L) {
    const u32x4 packed = mrow::pack8<T>(acc);
    u32x4* dst = reinterpret_cast<u32x4*>(t.out + r.b * t.o_sb + r.j * t.o_sj + lane * 8);
    __builtin_nontemporal_store(packed, dst);
    if (t.out_lse && lane == 0) t.out_lse[r.b * t.ol_sb + r.j] = L;
}

// cp = CP <= 16 shards, known at compile time; In is the payload reader,
// Out the output element type.  The row's CP LSEs have a
// wave-uniform address and are read with scalar loads, so the weights are
// computed once per wavefront with no cross-lane step; the CP payload loads
// are issued first and are all in flight while the weights are formed.
// Rows whose every weight is nonzero (the common case) take the plain FMA
// path; a row with an empty shard zeroes that shard's payload first.
template <int CP, typename In, typename Out>
__global__ __launch_bounds__(kBlock) void merge_kernel(const void* attn, const float* lse, int32_t a_sb, int32_t a_sj,
                                                       int32_t a_ss, int32_t l_sb, int32_t l_sj, int32_t l_ss,
                                                       int32_t h_local, MergeTail t) {
    const int lane = threadIdx.x & 63;
    const Row r = row_of(h_local);

    // elements of the payload
    const int64_t orow = static_cast<int64_t>(r.b) * a_sb + static_cast<int64_t>(r.j) * a_sj + lane * 8;
    const float* lrow = lse + static_cast<int64_t>(r.b) * l_sb + static_cast<int64_t>(r.j) * l_sj;
    // Every kernel argument the addresses need is read above this point, in
    // one batch of scalar loads, rather than a second batch after the
    // payload loads are issued.
    __builtin_amdgcn_sched_barrier(0);
    float x[CP], sc[CP];
#pragma unroll
    for (int s = 0; s < CP; ++s) {
        x[s] = lrow[static_cast<int64_t>(s) * l_ss];
        if (In::kScaled) sc[s] = lrow[static_cast<int64_t>(s) * l_ss + t.sc_off];
    }
    typename In::row_t v[CP];
#pragma unroll
    for (int s = 0; s < CP; ++s) v[s] = In::load(attn, orow + static_cast<int64_t>(s) * a_ss);
    // Keep every load above this point: nothing that waits on them may be
    // scheduled before the last one is issued.
    __builtin_amdgcn_sched_barrier(0);

    float M = x[0];
#pragma unroll
    for (int s = 1; s < CP; ++s) M = fmaxf(M, x[s]);
    float w[CP];
    float S = 0.0f;
#pragma unroll
    for (int s = 0; s < CP; ++s) {
        w[s] = mrow::shard_weight(x[s], M, t.to_log2);
        S += w[s];
    }
    const float inv = mrow::inv_sum(S);
    bool dense = true;
#pragma unroll
    for (int s = 0; s < CP; ++s) {
        w[s] *= inv;
        if (In::kScaled) w[s] *= sc[s];
        dense = dense && (w[s] != 0.0f);
    }

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (dense) {
#pragma unroll
        for (int s = 0; s < CP; ++s) In::fma(acc, w[s], v[s]);
    } else {
#pragma unroll
        for (int s = 0; s < CP; ++s) mrow::fma8<In>(acc, w[s], v[s]);
    }
    store_row<Out>(t, r, lane, acc, mrow::merged_lse(M, S, t.from_log2));
}

// 16 < cp <= 64: W wavefronts per row, wavefront w holding shards
// [16w, 16w + 16) of it, so that all of a row's loads are in flight at once
// (a row has few enough shards per wavefront, and rows enough wavefronts, to
// fill the chip even at small B).  Every wavefront forms the row's M, S and
// 1/S itself (mrow::lane_max_sum: a DPP tree over the shards) and the sum of
// its 16 shards, which is one accumulation group of the shared arithmetic,
// all wavefronts at once; after one barrier wavefront 0 adds the groups'
// sums (exact fp32 values in LDS) in ascending order and stores the row.  The
// result is merge_row_any's, bit for bit.  A block of kWavesPerBlock
// wavefronts holds kWavesPerBlock / W rows; spare rows of the last group
// repeat row h_local - 1 (same reads, same bits to the same place).
template <int W, typename In, typename Out>
__global__ __launch_bounds__(kBlock) void merge_kernel_wide(const void* attn, const float* lse, int32_t a_sb,
                                                            int32_t a_sj, int32_t a_ss, int32_t l_sb, int32_t l_sj,
                                                            int32_t l_ss, int32_t h_local, MergeTail t) {
    constexpr int kRows = kWavesPerBlock / W;
    constexpr int kPer = mrow::kAccGroup;  // shards per wavefront: one accumulation group
    __shared__ float hand[kRows][W][8][64];
    const int lane = threadIdx.x & 63;
    const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ri = v / W, w = v - ri * W;
    Row r;
    r.b = blockIdx.y;
    const int jr = blockIdx.x * kRows + ri;
    r.j = jr < h_local ? jr : h_local - 1;
    const int cp = t.cp;
    const int64_t orow = static_cast<int64_t>(r.b) * a_sb + static_cast<int64_t>(r.j) * a_sj + lane * 8;
    const float* lrow = lse + static_cast<int64_t>(r.b) * l_sb + static_cast<int64_t>(r.j) * l_sj;
    const int s0 = w * kPer;
    // Lane s holds shard s's LSE (and factor); they are loaded with the
    // payload, in the same memory round trip.
    const float x = mrow::lane_lse(lrow, l_ss, 0, cp);
    const float sc = In::kScaled && lane < cp ? lrow[static_cast<int64_t>(lane) * l_ss + t.sc_off] : 0.0f;
    typename In::row_t vals[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) vals[i] = In::load(attn, orow + static_cast<int64_t>(min(s0 + i, cp - 1)) * a_ss);
    __builtin_amdgcn_sched_barrier(0);

    // M, S and 1/S over all cp shards (mrow::lane_max_sum, cp <= 64).
    float M, S;
    mrow::lane_max_sum(x, cp, t.to_log2, M, S);
    float wl = mrow::shard_weight(x, M, t.to_log2) * mrow::inv_sum(S);
    if (In::kScaled) wl *= sc;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (s0 + i < cp) mrow::fma8<In>(acc, mrow::lane_value(wl, s0 + i), vals[i]);
    if (w > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hand[ri][w][i][lane] = acc[i];
    }
    __syncthreads();
    if (w == 0) {
        for (int k = 1; k < W && k * kPer < cp; ++k) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = acc[i] + hand[ri][k][i][lane];
        }
        store_row<Out>(t, r, lane, acc, mrow::merged_lse(M, S, t.from_log2));
    }
}

// 16 < cp <= 64, one wavefront per row: merge_row_any over the cp parts, 16
// at a time, the next 16 loads issued before the current FMAs.  Used for the
// MLA decode's split partials (scaled fp16): there the rows are many (every
// head of every shard) and a part's rows are adjacent in memory, so a block's
// four wavefronts, which take four adjacent rows, read 4 KiB runs of each
// part -- measured faster than spreading a row over several wavefronts
// (64 parts x 512 rows: 8.4 us against 10.4 us).
template <typename In, typename Out>
__global__ __launch_bounds__(kBlock) void merge_kernel_any(const void* attn, const float* lse, int32_t a_sb,
                                                           int32_t a_sj, int32_t a_ss, int32_t l_sb, int32_t l_sj,
                                                           int32_t l_ss, int32_t h_local, MergeTail t) {
    const int lane = threadIdx.x & 63;
    const Row r = row_of(h_local);
    const int64_t orow = static_cast<int64_t>(r.b) * a_sb + static_cast<int64_t>(r.j) * a_sj + lane * 8;
    const float* lrow = lse + static_cast<int64_t>(r.b) * l_sb + static_cast<int64_t>(r.j) * l_sj;
    float acc[8], M, S;
    mrow::merge_row_any<16, In>(attn, orow, a_ss, lrow, l_ss, t.sc_off, t.cp, t.to_log2, acc, M, S);
    store_row<Out>(t, r, lane, acc, mrow::merged_lse(M, S, t.from_log2));
}

// The MLA decode's split reduction and its shard merge in one launch
// (dcp_mla_decode_merged with DCP_FUSE_REDUCTIONS): wavefront (hi, s) of a
// block reduces the key splits of shard s of head h = kRmWaves / cp * x + hi
// (merge_row_any over the scaled fp16 partials, as merge_kernel_any and
// merge_kernel<n> do), stores that row of o_part / lse_part, and leaves it,
// rounded to the output type as stored, with its LSE in LDS; after the
// barrier wavefront (hi, 0) merges the head's cp rows from LDS into out /
// out_lse with merge_kernel<CP>'s arithmetic (sequential maximum and sum,
// normalised weights, FMAs in ascending shard order).  Every value is the one
// the separate launches compute and read back, so the bits are theirs; what
// is saved is the shard merge's launch and its re-read of o_part.  cp <= 16
// (the host checks): a block holds hb heads, hb * cp <= kRmWaves wavefronts.
constexpr int kRmWaves = 16;

template <typename Out>
__global__ __launch_bounds__(64 * kRmWaves) void reduce_merge_kernel(MergeArgs r, MergeArgs m, int32_t hq,
                                                                      int32_t hb) {
    typedef Payload16<F16, false, true> In;   // the split partials
    typedef Payload16<Out, false> Shard;      // a shard's row as stored in o_part
    __shared__ u32x4 rows[kRmWaves][64];
    __shared__ float lses[kRmWaves];
    const int cp = m.cp;
    const int lane = threadIdx.x & 63;
    const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hi = v / cp, s = v - hi * cp;
    const int b = blockIdx.y;
    const bool active = hi < hb;
    const int h0 = blockIdx.x * hb + hi;
    const int h = h0 < hq ? h0 : hq - 1;  // spare heads of the last block repeat the last one: same bits, same place
    if (active) {
        const int64_t j = static_cast<int64_t>(s) * hq + h;  // the row of o_part / lse_part within the token
        float acc[8], M, S;
        mrow::merge_row_any<8, In>(r.attn, b * r.a_sb + j * r.a_sj + lane * 8, r.a_ss, r.lse + b * r.l_sb + j * r.l_sj,
                                   r.l_ss, r.sc_off, r.cp, r.to_log2, acc, M, S);
        const u32x4 packed = mrow::pack8<Out>(acc);
        const float L = mrow::merged_lse(M, S, r.from_log2);
        __builtin_nontemporal_store(packed, reinterpret_cast<u32x4*>(r.out + b * r.o_sb + j * r.o_sj + lane * 8));
        if (lane == 0) r.out_lse[b * r.ol_sb + j] = L;
        rows[v][lane] = packed;
        if (lane == 0) lses[v] = L;
    }
    __syncthreads();
    if (!active || s != 0) return;
    const int v0 = hi * cp;
    float M = lses[v0];
    for (int t = 1; t < cp; ++t) M = fmaxf(M, lses[v0 + t]);
    float S = 0.0f;
    for (int t = 0; t < cp; ++t) S += mrow::shard_weight(lses[v0 + t], M, m.to_log2);
    const float inv = mrow::inv_sum(S);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < cp; ++t)
        mrow::fma8<Shard>(acc, mrow::shard_weight(lses[v0 + t], M, m.to_log2) * inv, rows[v0 + t][lane]);
    __builtin_nontemporal_store(mrow::pack8<Out>(acc), reinterpret_cast<u32x4*>(m.out + b * m.o_sb + h * m.o_sj + lane * 8));
    if (m.out_lse && lane == 0) m.out_lse[b * m.ol_sb + h] = mrow::merged_lse(M, S, m.from_log2);
}

typedef void (*MergeKernel)(const void*, const float*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                            MergeTail);

// The strides go to the kernel as 32-bit values: the planners check them
// with merge_strides_fit before anything is enqueued.
void launch_merge(MergeKernel k, const MergeArgs& a, dim3 grid, hipStream_t stream) {
    k<<<grid, dim3(kBlock), 0, stream>>>(a.attn, a.lse, static_cast<int32_t>(a.a_sb), static_cast<int32_t>(a.a_sj),
                                         static_cast<int32_t>(a.a_ss), static_cast<int32_t>(a.l_sb),
                                         static_cast<int32_t>(a.l_sj), static_cast<int32_t>(a.l_ss), a.h_local,
                                         tail_of(a));
}

template <int CP, typename In, typename Out>
void launch_fixed(const MergeArgs& a, dim3 grid, hipStream_t stream) {
    launch_merge(merge_kernel<CP, In, Out>, a, grid, stream);
}

template <int W, typename In, typename Out>
void launch_wide(const MergeArgs& a, dim3 grid, hipStream_t stream) {
    constexpr int kRows = kWavesPerBlock / W;
    launch_merge(merge_kernel_wide<W, In, Out>, a, dim3((a.h_local + kRows - 1) / kRows, grid.y), stream);
}

template <typename In, typename Out>
void launch_typed(const MergeArgs& a, dim3 grid, hipStream_t stream) {
    switch (a.cp) {
        case 1: launch_fixed<1, In, Out>(a, grid, stream); break;
        case 2: launch_fixed<2, In, Out>(a, grid, stream); break;
        case 3: launch_fixed<3, In, Out>(a, grid, stream); break;
        case 4: launch_fixed<4, In, Out>(a, grid, stream); break;
        case 5: launch_fixed<5, In, Out>(a, grid, stream); break;
        case 6: launch_fixed<6, In, Out>(a, grid, stream); break;
        case 7: launch_fixed<7, In, Out>(a, grid, stream); break;
        case 8: launch_fixed<8, In, Out>(a, grid, stream); break;
        case 9: launch_fixed<9, In, Out>(a, grid, stream); break;
        case 10: launch_fixed<10, In, Out>(a, grid, stream); break;
        case 11: launch_fixed<11, In, Out>(a, grid, stream); break;
        case 12: launch_fixed<12, In, Out>(a, grid, stream); break;
        case 13: launch_fixed<13, In, Out>(a, grid, stream); break;
        case 14: launch_fixed<14, In, Out>(a, grid, stream); break;
        case 15: launch_fixed<15, In, Out>(a, grid, stream); break;
        case 16: launch_fixed<16, In, Out>(a, grid, stream); break;
        default:
            if constexpr (In::kScaled) {
                launch_merge(merge_kernel_any<In, Out>, a, grid, stream);
            } else {
                if (a.cp <= 32)
                    launch_wide<2, In, Out>(a, grid, stream);
                else
                    launch_wide<4, In, Out>(a, grid, stream);
            }
            break;
    }
}

template <bool NT>
void launch_policy(const MergeArgs& a, dim3 grid, hipStream_t stream) {
    const bool f16_out = a.dtype == DCP_DTYPE_FP16;
    if (a.in_dtype == kPayloadF16Scaled) {
        if (f16_out)
            launch_typed<Payload16<F16, NT, true>, F16>(a, grid, stream);
        else
            launch_typed<Payload16<F16, NT, true>, Bf16>(a, grid, stream);
    } else if (f16_out) {
        launch_typed<Payload16<F16, NT>, F16>(a, grid, stream);
    } else {
        launch_typed<Payload16<Bf16, NT>, Bf16>(a, grid, stream);
    }
}

hipError_t launch(const MergeArgs& a, hipStream_t stream) {
    const int tokens = a.rows / a.h_local;
    const dim3 grid((a.h_local + kWavesPerBlock - 1) / kWavesPerBlock, tokens);
    if (a.cached)
        launch_policy<false>(a, grid, stream);
    else
        launch_policy<true>(a, grid, stream);
    return hipGetLastError();
}

}  // namespace

int merge_launch(const MergeArgs& a, void* stream) {
    return static_cast<int>(launch(a, static_cast<hipStream_t>(stream)));
}

int merge_launch_all(const MergeArgs& m, int64_t B, void* stream) {
    int64_t chunk = (int64_t{1} << 30) / m.h_local;
    if (chunk > kMaxLaunchTokens) chunk = kMaxLaunchTokens;
    for (int64_t t0 = 0; t0 < B; t0 += chunk) {
        const int64_t n = B - t0 < chunk ? B - t0 : chunk;
        const hipError_t e = launch(merge_args_at(m, t0, n), static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return static_cast<int>(e);
    }
    return 0;
}

int reduce_merge_launch(const MergeArgs& r, const MergeArgs& m, int64_t B, int hq, void* stream) {
    // One head (cp wavefronts) per block: measured against two and four heads
    // per block (producer B = 1, 64 splits: 64.0 against 66.9 and 74.0 us per
    // call) -- more blocks in flight beat the longer runs of adjacent rows.
    const int hb = 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int64_t t0 = 0; t0 < B; t0 += kMaxLaunchTokens) {
        const int64_t n = B - t0 < kMaxLaunchTokens ? B - t0 : kMaxLaunchTokens;
        const MergeArgs rc = merge_args_at(r, t0, n), mc = merge_args_at(m, t0, n);
        const dim3 grid((hq + hb - 1) / hb, static_cast<unsigned>(n));
        if (m.dtype == DCP_DTYPE_FP16)
            reduce_merge_kernel<F16><<<grid, dim3(64 * hb * m.cp), 0, st>>>(rc, mc, hq, hb);
        else
            reduce_merge_kernel<Bf16><<<grid, dim3(64 * hb * m.cp), 0, st>>>(rc, mc, hq, hb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return static_cast<int>(e);
    }
    return 0;
}

}  // namespace dcp

extern "C" int dcp_lse_combine(dcp_workspace* ws, const void* attn, int64_t B, int H, int64_t attn_sb,
                               int64_t attn_sh, const float* lse, int lse_layout, int64_t l0, int64_t l1, int64_t l2,
                               int lse_mode, void* out, int64_t out_sb, int64_t out_sh, float* out_lse,
                               int64_t out_lse_sb, void* hip_stream) {
    dcp::MergePlan plan;
    const int rc = dcp::plan_merge(ws, attn, B, H, attn_sb, attn_sh, lse, lse_layout, l0, l1, l2, lse_mode, out,
                                   out_sb, out_sh, out_lse, out_lse_sb, hip_stream, &plan);
    if (rc != DCP_OK) return rc;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    for (int64_t k = 0; k < plan.n_chunks; ++k) {
        const hipError_t e = dcp::launch(dcp::chunk_args(plan, k), stream);
        if (e != hipSuccess)
            return dcp::fail(DCP_ERR_HIP, "dcp_lse_combine: launch of chunk %lld of %lld failed: %s", (long long)k,
                             (long long)plan.n_chunks, hipGetErrorString(e));
    }
    return dcp::ok();
}
