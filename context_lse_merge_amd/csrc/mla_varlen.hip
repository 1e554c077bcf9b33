// mla_varlen.hip -- the work plan and the split reduction of the
// variable-length MLA decode (dcp_mla_partial_decode_varlen).
//
// In a decode batch every token (request) attends over its own number of
// cached rows, and the decode lengths decide which DCP shards are empty
// ("[Attention] Add direct symmetric-memory DCP A2A", vLLM PR #48897, amended
// port commit).  The lengths live on the device, so the host cannot size the
// key splits: a split length fixed from the longest possible token leaves
// most of the chip idle while the few long tokens finish.  Here a planning
// kernel sizes the splits from the actual lengths instead:
//  * one workgroup (its threads spread over the (token, shard) pairs, all
//    in exact 32-bit arithmetic) sums the key tiles of every pair (token, row
//    block, shard), picks st = max(ceil(total / 256), 8) tiles per split -- about
//    one split per compute unit over the whole batch, none shorter than 256
//    keys -- and gives each pair ceil(tiles / st) splits (one if it has at
//    most st tiles, including the empty pairs, which still write 0 / -inf);
//  * the work list is ordered longest split first (a counting sort over 1024
//    size bins): workgroups are dispatched in block order, so the long
//    splits start first and the short ones fill in behind them, the
//    longest-processing-time-first order of list scheduling;
//  * a pair with a single split writes its output straight into o_part /
//    lse_part; a pair with several leaves one normalised partial per split
//    in consecutive slots (fp16, each row scaled by a power of two whose
//    inverse is stored beside its LSE), and the reduction kernel below
//    merges them.
// The reduction is the merge's own row arithmetic (merge_row.h: the row
// maximum, the sum in its fixed order, normalised weights times the rows'
// scale factors, fp32 FMAs in ascending split order within groups of 16
// splits, the groups' sums added in order), so a pair split at the same
// boundaries gives the same bits on either path.  Which
// workgroup runs which split, and which slots a pair gets, depend on the
// order of LDS atomics; the arithmetic of a split does not, so the results
// are deterministic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dcp_internal.h"
#include "merge_row.h"

namespace dcp {
namespace {

constexpr int kBins = kMlaPlanThreads;
constexpr int kReduceWaves = 4;

__device__ __forceinline__ int32_t token_len(const MlaArgs& a, int32_t b) {
    const int32_t L = a.seq_lens[b];
    const int32_t T = static_cast<int32_t>(a.T);  // at most kVarlenMaxLen
    return L < 0 ? 0 : (L > T ? T : L);
}

// One workgroup of kMlaPlanThreads threads; thread i takes the (token,
// shard) pairs i, i + kMlaPlanThreads, ... (all row blocks of a token share
// them).  Pass 1 sums the tiles, pass 2 counts the splits per size bin, a
// scan turns the counts into the first list position of each bin (largest
// bin first), pass 3 places the splits.
__global__ __launch_bounds__(kMlaPlanThreads) void varlen_plan_kernel(MlaArgs a) {
    __shared__ unsigned long long s_total;
    __shared__ int32_t s_pos[kBins];
    __shared__ int32_t s_scan[2][kBins];
    __shared__ int32_t s_slots, s_split;
    const int tid = threadIdx.x;
    const int32_t cp = a.cp, rbt = a.rb_per_token;
    const int32_t n_ts = (a.rows / a.hq) * cp;  // (token, shard) pairs
    const bool il = a.interleaved != 0;
    if (tid == 0) {
        s_total = 0;
        s_slots = 0;
        s_split = 0;
    }
    s_pos[tid] = 0;
    __syncthreads();

    unsigned long long mine = 0;
    for (int32_t i = tid; i < n_ts; i += kMlaPlanThreads) {
        const int32_t b = i / cp;
        mine += varlen_shard_tiles(token_len(a, b), i - b * cp, cp, il);
    }
    if (mine) atomicAdd(&s_total, mine * rbt);
    __syncthreads();
    const int32_t st = varlen_split_tiles(static_cast<int64_t>(s_total));

    for (int32_t i = tid; i < n_ts; i += kMlaPlanThreads) {
        const int32_t b = i / cp;
        const int32_t t = varlen_shard_tiles(token_len(a, b), i - b * cp, cp, il);
        const int32_t n = varlen_splits(t, st);
        if (n > 1) atomicAdd(&s_pos[kBins - 1], (n - 1) * rbt);
        atomicAdd(&s_pos[varlen_bin(t - (n - 1) * st, st)], rbt);
    }
    __syncthreads();

    // Exclusive scan over the bins from the largest down: entry i of the scan
    // is bin kBins - 1 - i.
    const int32_t count = s_pos[kBins - 1 - tid];
    s_scan[0][tid] = count;
    __syncthreads();
    int src = 0;
    for (int d = 1; d < kBins; d *= 2) {
        const int32_t v = s_scan[src][tid] + (tid >= d ? s_scan[src][tid - d] : 0);
        s_scan[src ^ 1][tid] = v;
        src ^= 1;
        __syncthreads();
    }
    const int32_t inclusive = s_scan[src][tid];
    s_pos[kBins - 1 - tid] = inclusive - count;
    __syncthreads();

    for (int32_t i = tid; i < n_ts; i += kMlaPlanThreads) {
        const int32_t b = i / cp, s = i - b * cp;
        const int32_t t = varlen_shard_tiles(token_len(a, b), s, cp, il);
        const int32_t n = varlen_splits(t, st);
        const int bin = varlen_bin(t - (n - 1) * st, st);
        for (int32_t r = 0; r < rbt; ++r) {
            const int32_t q = (b * rbt + r) * cp + s;
            int32_t first = -1;
            if (n > 1) {
                first = atomicAdd(&s_slots, n);
                a.vl_splits[atomicAdd(&s_split, 1)] = VarlenSplit{q, first, n, 0};
                const int32_t pos = atomicAdd(&s_pos[kBins - 1], n - 1);
                for (int32_t p = 0; p < n - 1; ++p) a.vl_items[pos + p] = VarlenItem{q, p, first + p, 0};
            }
            const int32_t pos = atomicAdd(&s_pos[bin], 1);
            a.vl_items[pos] = VarlenItem{q, n - 1, first < 0 ? -1 : first + n - 1, 0};
        }
    }
    if (tid == kBins - 1) {
        // The last scan entry is the number of splits in all bins.
        a.vl_hdr->n_items = inclusive;
        a.vl_hdr->split_tiles = st;
    }
    __syncthreads();
    if (tid == 0) a.vl_hdr->n_split = s_split;
}

// Grid (kMlaRowsPerBlock / kReduceWaves, kVarlenTarget): block (x, y)
// merges rows 4x .. 4x + 3 of split pair y, one row per wavefront; lane l
// owns columns 8l .. 8l + 7.  Pairs past n_split exit.  Split p of row r sits
// in slot first + p: its fp16 row at part_o + ((first + p) * 128 + r) * 512,
// its LSE and scale at part_lse / part_scale + (first + p) * 128 + r.
template <typename Out>
__global__ __launch_bounds__(64 * kReduceWaves) void varlen_reduce_kernel(MlaArgs a, float to_log2,
                                                                           float from_log2) {
    const VarlenHeader* hdr = a.vl_hdr;
    if (static_cast<int>(blockIdx.y) >= hdr->n_split) return;
    const VarlenSplit sp = a.vl_splits[blockIdx.y];
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * kReduceWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_token = a.rb_per_token * a.cp;
    const int b = sp.pair / per_token;
    const int rem = sp.pair - b * per_token;
    const int rbi = rem / a.cp;
    const int s = rem - rbi * a.cp;
    const int h = rbi * kMlaRowsPerBlock + r;
    if (h >= a.hq) return;

    const int64_t row0 = static_cast<int64_t>(sp.first) * kMlaRowsPerBlock + r;  // slot `first`, row r
    const int64_t sc_off = a.part_scale - a.part_lse;
    float acc[8], M, S;
    mrow::merge_row_any<8, mrow::Payload16<mrow::F16, false, true>>(
        a.part_o, row0 * kMlaVDim + 8 * lane, static_cast<int64_t>(kMlaRowsPerBlock) * kMlaVDim, a.part_lse + row0,
        kMlaRowsPerBlock, sc_off, sp.n, to_log2, acc, M, S);
    const int64_t u = static_cast<int64_t>(s) * a.hq + h;
    *reinterpret_cast<mrow::u32x4*>(a.o + b * a.o_sb + u * a.o_sh + 8 * lane) = mrow::pack8<Out>(acc);
    if (lane == 0) a.lse[b * a.lse_sb + u] = mrow::merged_lse(M, S, from_log2);
}

}  // namespace

int varlen_plan_launch(const MlaArgs& a, void* stream) {
    varlen_plan_kernel<<<dim3(1), dim3(kMlaPlanThreads), 0, static_cast<hipStream_t>(stream)>>>(a);
    return static_cast<int>(hipGetLastError());
}

int varlen_reduce_launch(const MlaArgs& a, void* stream) {
    // The partial LSEs are in the caller's base, as the merge kernel reads them.
    const bool base2 = a.lse_scale == 1.0f;
    const float to_log2 = base2 ? 1.0f : 1.4426950408889634f;
    const float from_log2 = base2 ? 1.0f : 0.6931471805599453f;
    const dim3 grid(kMlaRowsPerBlock / kReduceWaves, kVarlenTarget);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.dtype == DCP_DTYPE_FP16)
        varlen_reduce_kernel<mrow::F16><<<grid, dim3(64 * kReduceWaves), 0, s>>>(a, to_log2, from_log2);
    else
        varlen_reduce_kernel<mrow::Bf16><<<grid, dim3(64 * kReduceWaves), 0, s>>>(a, to_log2, from_log2);
    return static_cast<int>(hipGetLastError());
}

}  // namespace dcp
