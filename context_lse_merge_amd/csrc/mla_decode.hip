// mla_decode.hip -- the MLA split-KV decode that produces the DCP shard
// partials (o_part, lse_part) on gfx950, and the dcp_mla_partial_decode entry
// point.
//
// What it computes ("[DCP] Optimize shared Output, Query, and Indexer/Top-K via
// peer memory", sglang PR #32851, commit log: each DCP rank attends over the
// KV tokens it owns and returns the LSE with the output; "[Attention] Add
// direct symmetric-memory DCP A2A", vLLM PR #48897, review thread: head_dim =
// kv_lora_rank = 512): for query row (b, h) and the keys t of one shard,
//     z_t = scale * <q, k_t> over 576 columns,  O = softmax(z) . V,  lse = log sum exp z,
// with the value V the first 512 columns of the cached row.
//
// Mapping to CDNA4.  Every query token attends over the same cache, so one
// shard is a flash-attention pass over M = B*hq query rows: a dense
// contraction, run on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//  * A workgroup owns 64 query rows (16 per wavefront) and one key range (a
//    split of one shard).  Each wavefront keeps its 16 query rows in registers
//    for the whole kernel, as 18 MFMA operand fragments of 32 columns.
//  * Keys stream through LDS 32 at a time, twice: row-major (for q.k) and
//    transposed (value column-major, for p.v), so every MFMA operand is read
//    as contiguous 8- or 16-byte LDS words.  The next tile's global loads are
//    issued before the current tile's MFMAs.
//  * The wavefront computes S^T = K Q^T (A = K, B = Q^T) and O^T += V^T P^T
//    (A = V^T, B = P^T).  In this orientation a lane holds eight scores of
//    query row lane % 16 and, with the k index of p.v permuted the same way in
//    V^T and P^T, exactly the B operand of the p.v MFMA: no shuffle between
//    the two products, and the running max/sum of row lane % 16 sit in the
//    same lanes as that row's output accumulators.
//  * Online softmax in base 2 (scale * log2 e folded into one multiply); the
//    row max is a 4-lane reduction per tile, the row sum stays lane-partial
//    until the end.  p is rounded to bf16 for the p.v MFMA; the sum uses the
//    fp32 p.
//  * Split-KV: shards are split into key ranges so that about 256 workgroups
//    (one per compute unit) exist even at B = 1; each split leaves an fp32
//    partial (running max, running sum, unnormalised output) in the scratch
//    buffer and a second kernel reduces them.  With a single split the first kernel
//    writes the final bf16 output and LSE itself.
//  * Workgroups that share a key range are placed on the same XCD (block ids
//    are dealt round-robin over the 8 XCDs), so a KV tile is fetched from HBM
//    about once per XCD-L2 rather than once per workgroup.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kDqk = kMlaQkDim;                  // 576
constexpr int kDv = kMlaVDim;                    // 512
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kKeys = kMlaKeysPerTile;           // 32
constexpr int kKStride = kDqk + 8;               // padded LDS row of K (elements)
constexpr int kVStride = kKeys + 4;              // padded LDS row of V^T (elements)
constexpr int kQSteps = kDqk / 32;               // 18 fragments of 32 columns
constexpr int kDTiles = kDv / 16;                // 32 output tiles of 16 columns
constexpr int kChunks = kKeys * kDqk / 8;        // 16-byte pieces of one K tile
constexpr int kChunksPerThread = kChunks / kThreads;
constexpr int kXcds = 8;

static_assert(kRowsPerWave * kWaves == kMlaRowsPerBlock, "rows per workgroup");
static_assert(kChunks % kThreads == 0, "K tile pieces per thread");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct __align__(16) Smem {
    uint16_t k[kKeys * kKStride];  // K tile, row-major: key x 576 (+8 pad)
    uint16_t vt[kDv * kVStride];   // value part transposed: 512 x key (+4 pad)
};

__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Which (row block, shard, split) a workgroup computes.  Block ids are dealt
// round-robin over the XCDs; consecutive work items -- the row blocks of one
// key range -- are given to blocks of the same XCD.
struct Work {
    int rb, s, p;
};

__device__ __forceinline__ Work work_of(const MlaArgs& a) {
    const int n = gridDim.x;
    const int L = blockIdx.x;
    const int w = (n % kXcds == 0) ? (L % kXcds) * (n / kXcds) + L / kXcds : L;
    Work k;
    k.rb = w % a.row_blocks;
    const int kc = w / a.row_blocks;
    k.s = kc / a.nsplit;
    k.p = kc - k.s * a.nsplit;
    return k;
}

// Global -> registers: piece c = tid + kThreads*i of the K tile starting at
// key t0 is key c % kKeys, columns [8*(c / kKeys), +8).  Keys at or past k1
// re-read key k1 - 1 (their scores are masked).
__device__ __forceinline__ void load_tile(const MlaArgs& a, int64_t t0, int64_t k1, int tid,
                                          u32x4 (&r)[kChunksPerThread]) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        const int c = tid + kThreads * i;
        const int key = c % kKeys;
        const int col = 8 * (c / kKeys);
        int64_t t = t0 + key;
        t = t < k1 ? t : k1 - 1;
        r[i] = *reinterpret_cast<const u32x4*>(a.kv + t * a.kv_st + col);
    }
}

// Registers -> LDS, row-major and, for the 512 value columns, transposed.
__device__ __forceinline__ void store_tile(Smem& sm, int tid, const u32x4 (&r)[kChunksPerThread]) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        const int c = tid + kThreads * i;
        const int key = c % kKeys;
        const int col = 8 * (c / kKeys);
        *reinterpret_cast<u32x4*>(&sm.k[key * kKStride + col]) = r[i];
        if (col < kDv) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.vt[(col + 2 * e) * kVStride + key] = static_cast<uint16_t>(r[i][e] & 0xFFFFu);
                sm.vt[(col + 2 * e + 1) * kVStride + key] = static_cast<uint16_t>(r[i][e] >> 16);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void mla_decode_kernel(MlaArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;  // query row of this lane within the wavefront
    const int g = lane >> 4;    // lane group: keys 4g..4g+3 of each 16-key half
    const Work wk = work_of(a);

    // Key range of this split of this shard.
    const int64_t s0 = (static_cast<int64_t>(wk.s) * a.T) / a.cp;
    const int64_t s1 = (static_cast<int64_t>(wk.s + 1) * a.T) / a.cp;
    const int64_t k0 = s0 + static_cast<int64_t>(wk.p) * a.split_len;
    const int64_t k1 = min(k0 + a.split_len, s1);

    // Query row of this lane (rows past the end repeat the last row and are not stored).
    const int row_raw = wk.rb * kMlaRowsPerBlock + wave * kRowsPerWave + r16;
    const int row = min(row_raw, a.rows - 1);
    const int b = row / a.hq;
    const int h = row - b * a.hq;

    // Q fragments: fragment f holds columns 32f + 8g .. +7 of this lane's row.
    bf16x8 qf[kQSteps];
    {
        const uint16_t* qrow = a.q + b * a.q_sb + h * a.q_sh + 8 * g;
#pragma unroll
        for (int f = 0; f < kQSteps; ++f) qf[f] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * f));
    }

    f32x4 oacc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of row r16, log2 units
    float l_run = 0.0f;       // lane-partial running sum of row r16

    u32x4 pre[kChunksPerThread];
    if (k0 < k1) load_tile(a, k0, k1, tid, pre);

    for (int64_t t0 = k0; t0 < k1; t0 += kKeys) {
        __syncthreads();  // the previous tile's LDS reads are done
        store_tile(sm, tid, pre);
        __syncthreads();
        if (t0 + kKeys < k1) load_tile(a, t0 + kKeys, k1, tid, pre);

        // S^T = K Q^T for keys [t0, t0+16) and [t0+16, t0+32): lane holds
        // scores of row r16 with keys 4g+i and 16+4g+i.
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* ka = &sm.k[r16 * kKStride + 8 * g];
        const uint16_t* kb = &sm.k[(16 + r16) * kKStride + 8 * g];
#pragma unroll
        for (int f = 0; f < kQSteps; ++f) {
            const bf16x8 fa = as_bf16x8(*reinterpret_cast<const u32x4*>(ka + 32 * f));
            const bf16x8 fb = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + 32 * f));
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, qf[f], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, qf[f], sb, 0, 0, 0);
        }

        // Online softmax (base 2) for row r16 over this tile.
        float z[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = (t0 + 4 * g + i < k1) ? sa[i] * a.scale_log2 : -INFINITY;
            z[4 + i] = (t0 + 16 + 4 * g + i < k1) ? sb[i] * a.scale_log2 : -INFINITY;
        }
        float tmax = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
        tmax = xor_max(tmax, 16);
        tmax = xor_max(tmax, 32);
        const float m_new = fmaxf(m_run, tmax);            // finite: the tile has a valid key
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
        float psum = 0.0f;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(z[i] - m_new);
            psum += p;
            pb[i] = static_cast<__bf16>(p);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // O^T += V^T P^T: output tile t is columns [16t, 16t+16); the k index
        // runs over keys 4g..4g+3 and 16+4g..16+4g+3, in P^T (pb) and V^T alike.
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
            const uint16_t* vrow = &sm.vt[(16 * t + r16) * kVStride];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 4 * g);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 + 4 * g);
            const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[t] * alpha, 0, 0, 0);
        }
    }

    // Row sums across the four lane groups; every lane of a row ends with the same l.
    const float l_tot = (l_run + __shfl_xor(l_run, 16, 64)) + (__shfl_xor(l_run, 32, 64) + __shfl_xor(l_run, 48, 64));
    if (row_raw >= a.rows) return;

    if (a.nsplit == 1) {
        // Final output: O / l in bf16, LSE in the caller's base; an empty shard gives 0 and -inf.
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = a.o + b * a.o_sb + (static_cast<int64_t>(wk.s) * a.hq + h) * a.o_sh + 4 * g;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
            const uint32_t lo = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(oacc[t][0] * inv))) |
                                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(oacc[t][1] * inv))) << 16);
            const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(oacc[t][2] * inv))) |
                                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(oacc[t][3] * inv))) << 16);
            *reinterpret_cast<u32x2*>(orow + 16 * t) = u32x2{lo, hi};
        }
        if (g == 0)
            a.lse[b * a.lse_sb + static_cast<int64_t>(wk.s) * a.hq + h] =
                l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * a.lse_scale : -INFINITY;
    } else {
        // Split partial: unnormalised fp32 output, running max and sum.
        const int64_t part = (static_cast<int64_t>(wk.s) * a.nsplit + wk.p) * a.rows + row;
        float* prow = a.part_o + part * kDv + 4 * g;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) *reinterpret_cast<f32x4*>(prow + 16 * t) = oacc[t];
        if (g == 0) {
            a.part_ml[2 * part] = l_tot > 0.0f ? m_run : -INFINITY;
            a.part_ml[2 * part + 1] = l_tot;
        }
    }
}

// Reduce the nsplit partials of every (shard, row): one wavefront per row,
// lane l owning columns [8l, 8l+8).  Grid: x = row groups of 4, y = shard.
// M = max_p m_p, w_p = 2^(m_p - M), L = sum_p w_p l_p, O = sum_p w_p O_p / L,
// in ascending p.  An all-empty row gives O = 0 and LSE = -inf.
__global__ __launch_bounds__(256) void mla_split_reduce_kernel(MlaArgs a) {
    const int lane = threadIdx.x & 63;
    const int row_raw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int row = __builtin_amdgcn_readfirstlane(min(row_raw, a.rows - 1));
    const int s = blockIdx.y;
    const int64_t base = static_cast<int64_t>(s) * a.nsplit * a.rows + row;  // part index of split 0

    float M = -INFINITY;
    for (int p = 0; p < a.nsplit; ++p) M = fmaxf(M, a.part_ml[2 * (base + static_cast<int64_t>(p) * a.rows)]);
    float L = 0.0f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int p = 0; p < a.nsplit; ++p) {
            const int64_t part = base + static_cast<int64_t>(p) * a.rows;
            const float m = a.part_ml[2 * part];
            if (m == -INFINITY) continue;  // empty split: its output is never read
            const float w = __builtin_amdgcn_exp2f(m - M);
            L += w * a.part_ml[2 * part + 1];
            const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + part * kDv + 8 * lane);
            const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] = fmaf(w, x0[i], acc[i]);
                acc[4 + i] = fmaf(w, x1[i], acc[4 + i]);
            }
        }
    }
    if (row_raw >= a.rows) return;
    const int b = row / a.hq;
    const int h = row - b * a.hq;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        packed[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[2 * i] * inv))) |
                    (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[2 * i + 1] * inv))) << 16);
    uint16_t* orow = a.o + b * a.o_sb + (static_cast<int64_t>(s) * a.hq + h) * a.o_sh + 8 * lane;
    *reinterpret_cast<u32x4*>(orow) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    if (lane == 0)
        a.lse[b * a.lse_sb + static_cast<int64_t>(s) * a.hq + h] =
            L > 0.0f ? (M + __builtin_amdgcn_logf(L)) * a.lse_scale : -INFINITY;
}

}  // namespace
}  // namespace dcp

extern "C" int dcp_mla_partial_decode(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                                      int64_t kv_tokens, int64_t kv_st, int cp, float softmax_scale, int lse_mode,
                                      void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part, int64_t lse_sb,
                                      void* scratch, size_t scratch_bytes, void* hip_stream) {
    dcp::MlaPlan plan;
    const int rc = dcp::plan_mla(q, B, hq, q_sb, q_sh, kv, kv_tokens, kv_st, cp, softmax_scale, lse_mode, o_part,
                                 o_sb, o_sh, lse_part, lse_sb, scratch, scratch_bytes, &plan);
    if (rc != DCP_OK) return rc;
    if (plan.blocks == 0) return dcp::ok();
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    dcp::mla_decode_kernel<<<dim3(static_cast<unsigned>(plan.blocks)), dim3(dcp::kThreads), 0, stream>>>(plan.args);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && plan.args.nsplit > 1) {
        const dim3 grid((plan.args.rows + 3) / 4, plan.args.cp);
        dcp::mla_split_reduce_kernel<<<grid, dim3(256), 0, stream>>>(plan.args);
        e = hipGetLastError();
    }
    if (e != hipSuccess)
        return dcp::fail(DCP_ERR_HIP, "dcp_mla_partial_decode: launch failed: %s", hipGetErrorString(e));
    return dcp::ok();
}
