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
// contraction, run on MFMA (v_mfma_f32_16x16x32_bf16, or _f16 for fp16
// inputs; fp32 accumulate).
//  * A workgroup owns 128 query rows and one key range (a split of one
//    shard), with 8 wavefronts (two per SIMD, so one wavefront's softmax and
//    waits overlap the other's MFMAs).  The two products are split
//    differently: wavefront w computes the scores and the online softmax of
//    its own 16 query rows (kept in registers for the whole kernel as 18 MFMA
//    operand fragments of 32 columns), but accumulates p.v for 64 of the 512
//    value columns of all 128 rows.  Each wavefront publishes its rows' p (the
//    p.v operand, 1 KiB) and rescale factors in LDS, and every wavefront
//    reads all eight: a value fragment read from LDS then feeds eight MFMAs
//    instead of one, which cuts the p.v operand reads from 32 to 12 KiB per
//    wavefront and tile (the q.k reads stay 36 KiB).
//  * Keys stream through LDS 32 at a time in three buffers (one barrier per
//    tile).  Tiles are copied global -> LDS by the gfx950 direct loads
//    (global_load_lds_dwordx4), with no register staging; every tile but a
//    split's last is copied with a scalar base address and one per-lane
//    offset fixed for the whole kernel, so the copies cost no vector
//    instructions.  The scores of a tile are computed one interval before
//    its p.v, so a buffer is busy for two intervals and each copy is issued
//    one tile ahead, in two parts around the p.v (a copy holds the vector
//    memory unit for about 64 clocks, one per cache line and 16-lane pass).
//    With a single row block, where no other workgroup shares a key range in
//    the L2, scores and p.v of a tile share an interval (two barriers) and
//    two tiles are in flight instead.
//  * Q is loaded as 4 rows x 64 B per 16-lane pass and moved into the MFMA
//    operand layout with ds_bpermute; the epilogue regroups each row's pieces
//    over its four lane groups (permlane swaps) so that every lane stores
//    16-byte words.
//  * LDS layout of a tile: 36 blocks of 1 KiB, block (h, b) holding the 16-byte
//    chunks 4b..4b+3 of keys 16h..16h+15, chunk c of key k at slot
//    16 (c % 4) + ((k % 16) ^ 8 (b % 2)).  Measured on gfx950, a 16-byte LDS
//    read runs at the full 256 B/clk only when every 16-lane group of the
//    wavefront reads one 256-byte row in the same lane order, and the
//    transpose read only when each half-wavefront touches all 64 banks; in
//    this layout the q.k operand read of a 32-column step is exactly one
//    block read in one order (XOR-permuted alike in every group), and the
//    p.v operand pairs chunk c (XOR 0) with chunk c + 4 (XOR 8): the eight
//    keys a half-wavefront reads from the even block land on banks 0-31 and
//    those from the odd block on banks 32-63 (or the reverse), so every
//    transpose read is free of bank conflicts (counted: 0 conflict cycles;
//    XOR 4 left the two 16-lane groups of a half-wavefront on the same 32
//    banks, 1.28 conflict cycles per LDS instruction).  One direct copy fills
//    one block.
//  * The wavefront computes S^T = K Q^T (A = K, B = Q^T) and O^T += V^T P^T
//    (A = V^T, B = P^T).  In this orientation a lane holds eight scores of
//    query row lane % 16 and, with the k index of p.v permuted the same way in
//    V^T and P^T, exactly its share of the B operand of the p.v MFMA: the
//    exchange is a 16-byte LDS write per lane, and the reading wavefront's
//    lane l takes slot l, in the lane order that reads LDS at full rate.  The
//    q.k operand is read as 16-byte LDS words; the p.v operand, which needs
//    the value transposed, is read from the same row-major tile with the
//    transpose load
//    ds_read_b64_tr_b16: within each 16-lane group it returns lane j element
//    i of the 8-byte chunk lane 4i + j/4 pointed at, so lanes pointing at
//    V[key][d0 + 4(j%4)] of four keys receive a column of V^T.
//  * Online softmax in base 2 (scale * log2 e applied once to the tile
//    maximum and inside each exponent's FMA, p = 2^(s c - m) with one
//    rounding; a key mask only on a split's last, partial tile); the
//    row max is a 4-lane reduction per tile, the row sum stays lane-partial
//    until the end, and the reference maximum moves (rescaling the output
//    accumulators) only when some row's score exceeds it by more than 8
//    (log2 units), so p stays at most 256.  p is rounded to bf16 for the p.v MFMA; the sum
//    uses the fp32 p.
//  * Split-KV: shards are split into key ranges so that about 256 workgroups
//    (one per compute unit) exist even at B = 1; each split leaves its
//    normalised output (fp16, scaled per row by a power of two, the inverse
//    factor stored with the LSE) and its LSE in the scratch buffer, and the
//    merge kernel of dcp_lse_combine (its scaled-fp16 instance) reduces the
//    splits of each (token, shard, head) exactly as it merges DCP shards.  With a
//    single split the kernel writes the final output and LSE itself.  With
//    per-token lengths (seq_lens) the splits are sized on the device instead
//    and the workgroup runs one item of a work list (mla_varlen.hip).
//  * Workgroups that share a key range are placed on the same XCD (block ids
//    are dealt round-robin over the 8 XCDs), so a KV tile is fetched from HBM
//    about once per XCD-L2 rather than once per workgroup.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dcp_internal.h"
#include "merge_row.h"

namespace dcp {
namespace {

constexpr int kDqk = kMlaQkDim;                  // 576
constexpr int kDv = kMlaVDim;                    // 512
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kKeys = kMlaKeysPerTile;           // 32
constexpr int kRowChunks = kDqk / 8;             // 72 chunks of 16 bytes per K row
constexpr int kTileChunks = kKeys * kRowChunks;  // 2304 per tile
constexpr int kTileElems = kKeys * kDqk;
constexpr int kDmaPerTile = kTileChunks / 64;    // 36 wavefront-wide 1 KiB copies
constexpr int kQSteps = kDqk / 32;               // 18 fragments of 32 columns
constexpr int kXcds = 8;

static_assert(kRowsPerWave * kWaves == kMlaRowsPerBlock, "rows per workgroup");
static_assert(kTileChunks % 64 == 0, "a tile is whole 1 KiB wavefront copies");
static_assert(kRowChunks % 4 == 0 && (kDv / 8) % 8 == 0, "blocks of 4 chunks; p.v chunk pairs c, c + 4");
static_assert(kTileChunks == 64 * 2 * (kRowChunks / 4), "a tile is 2 x 18 blocks");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));  // the transpose load's fp16 vector type
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int kBlockElems = 512;                            // one 1 KiB LDS block
constexpr int kHalfBlocks = kRowChunks / 4;                  // 18 blocks per 16 keys
constexpr int kHalfElems = kHalfBlocks * kBlockElems;        // keys 16..31 start here

// Reductions over lane pairs (l, l ^ 16) and (l, l ^ 32) without an LDS round
// trip: v_permlane16_swap / v_permlane32_swap of a value with itself return
// the two rows (halves) of each pair, one in each result.
// max(a, b) of values that are never NaN here, as a bare v_max_f32: fmaxf
// would first pass each operand the compiler cannot prove canonical (a
// permlane result, say) through a NaN-quieting v_max_f32 x, x of its own.
// Only for operands written by ordinary vector instructions: an MFMA result
// needs wait states before it is read, which the compiler inserts only ahead
// of instructions it generates itself.
__device__ __forceinline__ float max_nn(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}


__device__ __forceinline__ float max_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// The two 16-bit element types of q, the cache and the output: the MFMA,
// the transpose load and the conversions of each.  Everything else in the
// kernel moves raw 16-bit words and is shared.
struct Bf16 {
    typedef __bf16 elem;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    typedef mrow::Bf16 merge_t;  // the same element type for the merges of the fused epilogue
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ v4 tr(const __attribute__((address_space(3))) char* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    }
};

struct F16 {
    typedef _Float16 elem;
    typedef f16x8 v8;
    typedef f16x4 v4;
    typedef mrow::F16 merge_t;
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ v4 tr(const __attribute__((address_space(3))) char* p) {
        return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(p)));
    }
};

template <typename T>
__device__ __forceinline__ typename T::v8 as_v8(u32x4 v) { return __builtin_bit_cast(typename T::v8, v); }

// Transpose load of 8 bytes at LDS element offset `off` of `base`.
template <typename T>
__device__ __forceinline__ typename T::v4 ds_read_tr(const uint16_t* base, int off) {
    return T::tr((const __attribute__((address_space(3))) char*)(base) + 2 * off);
}

// Round to nearest even in the element type, as raw bits.
template <typename T>
__device__ __forceinline__ uint32_t to_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<typename T::elem>(x));
}

// Which (row block, shard, split) a workgroup computes.  Block ids are dealt
// round-robin over the XCDs; consecutive work items -- the row blocks of one
// key range -- are given to blocks of the same XCD.
struct Work {
    int rb, s, p;
    int slot;  // variable length: partial slot, or -1 to write o_part directly
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
    k.slot = -1;
    return k;
}

// A value the compiler must treat as unknown: addresses derived from it are
// recomputed where they are used instead of being hoisted out of the key loop
// and kept (or spilled) across it -- registers are the scarce resource here.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// byte address lds + 16 l.  Issued as inline assembly so that the compiler
// does not track it: its automatic waits would otherwise stall every tile on
// the copies just issued (it cannot tell which LDS buffer they write).  The
// kernel therefore waits for these copies itself (vmcnt) before the barrier
// that publishes a tile; nothing else in the key loop issues vector memory
// instructions.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)(p)));
}

// The LDS address goes in M0, bound as an input operand so that the compiler
// writes M0 itself and knows it is in use; the s_nop keeps one wait state
// between that write and the copy that reads it.
__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}

constexpr int kDmaPerWave = (kDmaPerTile + kWaves - 1) / kWaves;  // copies per wavefront, at most
static_assert(kWaves * (kDmaPerWave - 2) + kWaves - 1 < kDmaPerTile, "all but a wavefront's last copy exist");
constexpr int kTileAlloc = kTileElems;

// The keys a workgroup visits: logical key j (0, 1, ... within its shard) is
// cache row rows0 + j * rstride elements (rstride = kv_st, or cp * kv_st when
// the shard owns every cp-th row).
struct KeyRows {
    const uint16_t* rows0;
    int32_t rstride;
};

// Copy the K tile of keys [t0, t0 + 32) into LDS tile `dst` with direct
// loads: copy n = w + 8 i (n < 36: wavefronts 0-3 issue five, 4-7 four) of
// wavefront w fills block n = 18 h + b, its lane l slot l, i.e. chunk
// 4b + l / 16 of key 16 h + ((l % 16) ^ 8 (b % 2)).  In a ragged last tile,
// keys at or past k1 re-read key k1 - 1 (their scores are masked).  Every
// wait for these copies is a wait for all of them (vmcnt(0)), so the counts
// may differ between wavefronts.
__device__ __forceinline__ void dma_tile(const KeyRows& kr, uint16_t* dst, int64_t t0, int64_t k1, int wave,
                                         int lane_in) {
    const uint16_t* base = kr.rows0 + t0 * kr.rstride;
    const int last = static_cast<int>(min(k1 - 1 - t0, static_cast<int64_t>(kKeys - 1)));
    const int lane = opaque(lane_in);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int n = wave + kWaves * i;
        if (i + 1 < kDmaPerWave || n < kDmaPerTile) {  // only the last copy can fall past block 35
            const int h = n >= kHalfBlocks ? 1 : 0;
            const int blk = n - h * kHalfBlocks;
            const int key = 16 * h + ((lane & 15) ^ (8 * (blk & 1)));
            const int chunk = 4 * blk + (lane >> 4);
            const int o = min(key, last) * kr.rstride + 8 * chunk;
            lds_dma16(base + o, lds_addr(dst + kBlockElems * n));
        }
    }
}

// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset: the address arithmetic stays scalar.
__device__ __forceinline__ void lds_dma16_s(const uint16_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Byte offset of lane `lane`'s 16 bytes within every block wavefront `wave`
// copies of a full tile: key (lane % 16) ^ 8 (b % 2), chunk lane / 16 of the
// block's four, and b % 2 = wave % 2 for every copy n = wave + 8 i of the
// wavefront (n % 18 and n have the same parity).  The key is at most 15 (the
// half's 16 rows go into the scalar base), so for row strides below
// kFullTileMaxStride elements the offset stays below 2^31.  The host limits
// the row stride to (2^31 - 576) / 32 elements, so validated calls always
// take this path; the check keeps the kernel's own assumption explicit.
constexpr int32_t kFullTileMaxStride = 1 << 26;
__device__ __forceinline__ uint32_t full_tile_lane_offset(int32_t rstride, int wave, int lane) {
    const int key = (lane & 15) ^ (8 * (wave & 1));
    return 2u * (static_cast<uint32_t>(key) * static_cast<uint32_t>(rstride) + 8u * static_cast<uint32_t>(lane >> 4));
}

// dma_tile for a tile whose 32 keys are all valid: block n = 18 h + b of the
// tile reads rows 16 h .. of it from 32 b elements on, a scalar offset; the
// lane's part is full_tile_lane_offset.  The same bytes as dma_tile.  Copies
// I0 .. I1 - 1 of the wavefront's (all of them by default).
template <int I0 = 0, int I1 = kDmaPerWave>
__device__ __forceinline__ void dma_tile_full(const KeyRows& kr, uint16_t* dst, int64_t t0, uint32_t lane_off,
                                              int wave) {
    const uint16_t* base = kr.rows0 + t0 * kr.rstride;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const int n = wave + kWaves * i;
        if (i + 1 < kDmaPerWave || n < kDmaPerTile) {  // only the last copy can fall past block 35
            const int h = n >= kHalfBlocks ? 1 : 0;
            const int blk = n - h * kHalfBlocks;
            lds_dma16_s(base + static_cast<int64_t>(16 * h) * kr.rstride + 32 * blk, lane_off,
                        lds_addr(dst + kBlockElems * n));
        }
    }
}

// Wait for all of this wavefront's tile copies, then synchronise.
__device__ __forceinline__ void all_tiles_ready() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
}

// Per-lane LDS offsets (elements, before the tile base) of the operands.
struct LaneOffsets {
    int s_even, s_odd;  // q.k operand of key r16, for fragment f even / odd, before + 512 f
    int tr[4];          // p.v operand (keys 0..15), output tile t with t % 4 == u, before + 1024 (t / 4)
};

// What the wavefronts of a workgroup exchange per key tile.  Wavefront w
// computes the scores and softmax of its own 16 query rows (row tile w) and
// publishes their p.v operand P^T -- lane l's eight 16-bit p at slot l of
// block w -- and, on a tile where its rows' reference maximum moved, the
// rescale factor of each of those rows.  The p.v product is split by output
// columns instead: wavefront w accumulates columns 64w .. 64w+63 of all 128
// rows, reading the eight P^T blocks.
struct TileExchange {
    u32x4 p[kWaves][64];
    float alpha[kMlaRowsPerBlock];
    uint8_t moved[kWaves];
};

// The running maximum of the online softmax lags the true one by at most
// this much (log2 units): p <= 2^8.
constexpr float kLazyLog2 = 8.0f;

// Scores and online softmax of this wavefront's 16 rows for one 32-key tile;
// publishes P^T and the rescale factors in `ex`.  kMask: the tile may hold
// keys at or past k1 (a split's last tile), whose scores are masked.
template <typename T, bool kMask>
__device__ __forceinline__ void qk_tile(const MlaArgs& a, const uint16_t* kt, const LaneOffsets& off,
                                        const typename T::v8 (&qf)[kQSteps], float& m_run, float& l_run, int64_t t0,
                                        int64_t k1, int g, int wave, int lane, TileExchange& ex) {
    // S^T = K Q^T for keys [t0, t0+16) (sa) and [t0+16, t0+32) (sb): the lane
    // holds the scores of row r16 with keys 4g+i and 16+4g+i.
    // Operand fragments are read kAhead steps before the MFMA that uses them
    // (a ring of kAhead + 1), and the scheduler is told to interleave the
    // reads with the MFMAs: without this every MFMA waits out a full LDS
    // latency.
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    {
        constexpr int kAhead = 2;
        typename T::v8 ra[kAhead + 1], rb[kAhead + 1];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < kQSteps + kAhead; ++f) {
            if (f < kQSteps) {
                const int o = ((f & 1) ? off.s_odd : off.s_even) + kBlockElems * f;
                ra[f % (kAhead + 1)] = as_v8<T>(*reinterpret_cast<const u32x4*>(kt + o));
                rb[f % (kAhead + 1)] = as_v8<T>(*reinterpret_cast<const u32x4*>(kt + o + kHalfElems));
            }
            if (f >= kAhead) {
                const int u = f - kAhead;
                sa = T::mfma(ra[u % (kAhead + 1)], qf[u], sa);
                sb = T::mfma(rb[u % (kAhead + 1)], qf[u], sb);
            }
        }
#pragma unroll
        for (int f = 0; f < kQSteps + kAhead; ++f) {
            if (f < kQSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
            if (f >= kAhead) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    float z[8];  // raw scores; the scale is applied in the exponent
    if (kMask) {
        const int rem = static_cast<int>(min(k1 - t0, static_cast<int64_t>(kKeys)));  // valid keys of the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = (4 * g + i < rem) ? sa[i] : -INFINITY;
            z[4 + i] = (16 + 4 * g + i < rem) ? sb[i] : -INFINITY;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = sa[i];
            z[4 + i] = sb[i];
        }
    }
    // fmaxf here: its operands are MFMA results, whose wait states before a
    // vector read the compiler inserts only for instructions it generates.
    float tmax = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
    tmax = max_xor32(max_xor16(tmax)) * a.scale_log2;  // finite: the tile has a valid key
    // Lazy rescaling: the running maximum m_run (the reference of the
    // exponentials) moves only when some row's tile maximum exceeds it by
    // more than kLazyLog2; otherwise the tile's p = 2^(z - m_run) stay below
    // 2^kLazyLog2 (safe in the 16-bit p and the fp32 sums), and O / l and
    // m_run + log2 l do not depend on which reference was used.  Rescaling
    // the accumulators then happens on the first tile of a split and rarely
    // after, instead of on every tile where some row's maximum grows.
    const bool moved = __any(tmax > m_run + kLazyLog2);
    if (moved) {
        const float m_new = max_nn(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile, 1 for unchanged rows
        l_run *= alpha;
        m_run = m_new;
        if (g == 0) ex.alpha[kRowsPerWave * wave + (opaque(lane) & 15)] = alpha;  // address formed here, not kept live
    }
    if (lane == 0) ex.moved[wave] = moved ? 1 : 0;
    float psum = 0.0f;
    typename T::v8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], a.scale_log2, -m_run));
        psum += p;
        pb[i] = static_cast<typename T::elem>(p);
    }
    l_run += psum;
    ex.p[wave][lane] = __builtin_bit_cast(u32x4, pb);
}

// O^T += V^T P^T for this wavefront's output columns and all 128 rows: output
// tile t = 4 wave + u holds value columns 8c..8c+7 and 8c+32..8c+39 with
// c = 8 wave + u (chunks c and c + 4), acc[rt][u] its rows 16 rt .. 16 rt + 15.
// The k index runs over keys 4g..4g+3 and 16+4g..16+4g+3, in P^T and V^T
// alike.  Rows whose reference maximum moved on this tile are rescaled first.
template <typename T>
__device__ __forceinline__ void pv_tile(const uint16_t* kt, const LaneOffsets& off, f32x4 (&acc)[kWaves][4],
                                        const TileExchange& ex, int wave, int lane) {
    const uint2 mvw = *reinterpret_cast<const uint2*>(ex.moved);
    typename T::v8 va[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int o = off.tr[u] + 2 * kBlockElems * wave;
        const typename T::v4 lo = ds_read_tr<T>(kt, o), hi = ds_read_tr<T>(kt, o + kHalfElems);
        va[u] = typename T::v8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const uint32_t m_lo = __builtin_amdgcn_readfirstlane(mvw.x), m_hi = __builtin_amdgcn_readfirstlane(mvw.y);
    if (m_lo | m_hi) {
#pragma unroll
        for (int rt = 0; rt < kWaves; ++rt) {
            const bool mv = (((rt < 4 ? m_lo : m_hi) >> (8 * (rt & 3))) & 0xffu) != 0;
            const float al = mv ? ex.alpha[kRowsPerWave * rt + (lane & 15)] : 1.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[rt][u] *= al;
        }
    }
    {
        constexpr int kAhead = 2;
        u32x4 pr[kAhead + 1];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < kWaves + kAhead; ++r) {
            if (r < kWaves) pr[r % (kAhead + 1)] = ex.p[r][lane];
            if (r >= kAhead) {
                const int q = r - kAhead;
                const typename T::v8 pf = as_v8<T>(pr[q % (kAhead + 1)]);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[q][u] = T::mfma(va[u], pf, acc[q][u]);
            }
        }
#pragma unroll
        for (int r = 0; r < kWaves + kAhead; ++r) {
            if (r < kWaves) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 P^T read
            if (r >= kAhead) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // 4 MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Where the rows of a workgroup go: query row rr (0..127) of the workgroup
// is (b, h), stored if valid.  One shared cache: rows of 128 consecutive
// (token, head) pairs; with seq_lens, heads h_base .. of token b_tok.
struct RowPlace {
    int rb, b_tok, h_base;
    bool varlen;
};

__device__ __forceinline__ void place_row(const MlaArgs& a, const RowPlace& rp, int rr, int& b, int& h, bool& valid) {
    if (rp.varlen) {
        const int h_raw = rp.h_base + rr;
        valid = h_raw < a.hq;
        b = rp.b_tok;
        h = min(h_raw, a.hq - 1);
    } else {
        const int row_raw = rp.rb * kMlaRowsPerBlock + rr;
        valid = row_raw < a.rows;
        const int row = min(row_raw, a.rows - 1);
        b = row / a.hq;
        h = row - b * a.hq;
    }
}

// Lane group g of a row holds, in d[t] (t = 0..3), the packed 16-bit values
// of columns 8t + 4 (g % 2) + 32 (g / 2) .. +3 of its wavefront's 64-column
// slice.  A 4 x 4 transpose of these 8-byte items over the row's four lane
// groups (lanes r16, r16 + 16, r16 + 32, r16 + 48; two permlane stages, all
// lanes active) leaves group g with columns 8g .. 8g + 7 in d[0], d[1] and
// 32 + 8g .. 32 + 8g + 7 in d[2], d[3]: each lane then stores two 16-byte
// words, and one store instruction writes 64 contiguous bytes of each of its
// 16 rows instead of two 16-byte pieces.
__device__ __forceinline__ void regroup_slice(uint32_t (&d)[4][2]) {
    // Groups g and g ^ 2: items 2 + t0 of groups 0, 1 trade places with items
    // t0 of groups 2, 3.
#pragma unroll
    for (int t0 = 0; t0 < 2; ++t0)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto p = __builtin_amdgcn_permlane32_swap(d[t0][w], d[2 + t0][w], false, false);
            d[t0][w] = p[0];
            d[2 + t0][w] = p[1];
        }
    // Groups g and g ^ 1: items 2c + 1 of the even groups trade places with
    // items 2c of the odd ones.
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto p = __builtin_amdgcn_permlane16_swap(d[2 * c][w], d[2 * c + 1][w], false, false);
            d[2 * c][w] = p[0];
            d[2 * c + 1][w] = p[1];
        }
}

// The epilogue: O / l and the LSE in the caller's base; an empty shard or
// split gives 0 and -inf.  Wavefront w stores columns 64w .. 64w+63 of all
// 128 rows, and the LSE (and scale) of its own row tile, whose softmax state
// it holds.  One split: the element type, straight into o_part / lse_part.
// Several: into the scratch -- as head p*cp*hq + s*hq + h, for the merge
// kernel to reduce over the splits, or with seq_lens as row rr of the item's
// slot, for the split reduction -- in fp16, the row multiplied by 2^k so that
// its largest magnitude lies in [2^14, 2^15) (fp16 then carries 11
// significant bits relative to the row's largest value), with 2^-k stored
// beside the LSE.  The row sums and the rows' largest magnitudes (per
// 64-column slice) travel through LDS.
template <typename T>
__device__ __forceinline__ void store_block(const MlaArgs& a, const Work& wk, const RowPlace& rp, int wave, int lane,
                                            const f32x4 (&acc)[kWaves][4], float m_run, float l_run, bool direct,
                                            float* lsum, float (*amaxp)[kMlaRowsPerBlock]) {
    const int r16 = lane & 15, g = lane >> 4;
    // Row sums across the four lane groups; every lane of a row ends with the same l.
    const float l_own = sum_xor32(sum_xor16(l_run));
    if (g == 0) lsum[kRowsPerWave * wave + r16] = l_own;
    if (!direct) {
#pragma unroll
        for (int rt = 0; rt < kWaves; ++rt) {
            float am = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(acc[rt][u][i]));
            am = max_xor32(max_xor16(am));
            if (g == 0) amaxp[wave][kRowsPerWave * rt + r16] = am;
        }
    }
    __syncthreads();
    // After regroup_slice this lane's columns are 64 wave + 8 g (+ 32).
    const int ocol = 64 * wave + 8 * g;
#pragma unroll
    for (int rt = 0; rt < kWaves; ++rt) {
        const int rr = kRowsPerWave * rt + r16;
        int b, h;
        bool valid;  // the same for the four lanes of a row: the regrouping stays within a row
        place_row(a, rp, rr, b, h, valid);
        const float l_tot = lsum[rr];
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const bool own = rt == wave;  // this wavefront's softmax rows: m_run is theirs
        const float lse = own && l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * a.lse_scale : -INFINITY;
        uint32_t d[4][2];
        uint16_t* orow;
        int64_t prow_idx = 0;  // partial row of the scratch
        int k = 0;
        if (direct) {
            const int64_t u = static_cast<int64_t>(wk.s) * a.hq + h;
            orow = a.o + b * a.o_sb + u * a.o_sh + ocol;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 v = acc[rt][t];
                d[t][0] = to_bits<T>(v[0] * inv) | (to_bits<T>(v[1] * inv) << 16);
                d[t][1] = to_bits<T>(v[2] * inv) | (to_bits<T>(v[3] * inv) << 16);
            }
        } else {
            float amax = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, amaxp[w][rr]);
            if (rp.varlen)
                prow_idx = static_cast<int64_t>(wk.slot) * kMlaRowsPerBlock + rr;
            else
                prow_idx = b * a.part_sb + (static_cast<int64_t>(wk.p) * a.cp + wk.s) * a.hq + h;
            // amax * inv = m 2^e with m in [0.5, 1): k = 15 - e.  Capped at 100
            // so that 2^-k stays a normal float (rows below 2^-85 keep fewer bits;
            // an all-zero row gets k = 15).  1/l <= 1, so inv * 2^k stays finite.
            k = min(15 - __builtin_amdgcn_frexp_expf(amax * inv), 100);
            const float mul = __builtin_amdgcn_ldexpf(inv, k);
            orow = a.part_o + prow_idx * kDv + ocol;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 v = acc[rt][t];
                d[t][0] = to_bits<F16>(v[0] * mul) | (to_bits<F16>(v[1] * mul) << 16);
                d[t][1] = to_bits<F16>(v[2] * mul) | (to_bits<F16>(v[3] * mul) << 16);
            }
        }
        regroup_slice(d);
        if (!valid) continue;
        *reinterpret_cast<u32x4*>(orow) = u32x4{d[0][0], d[0][1], d[1][0], d[1][1]};
        *reinterpret_cast<u32x4*>(orow + 32) = u32x4{d[2][0], d[2][1], d[3][0], d[3][1]};
        if (own && g == 0) {
            if (direct) {
                a.lse[b * a.lse_sb + static_cast<int64_t>(wk.s) * a.hq + h] = lse;
            } else {
                a.part_lse[prow_idx] = lse;
                a.part_scale[prow_idx] = __builtin_amdgcn_ldexpf(1.0f, -k);
            }
        }
    }
}


// Count this workgroup into *cnt, one of n arrivals, and tell whether it was
// the last.  Each wavefront first waits until its own stores have completed
// (vmcnt counts stores too), the workgroup synchronises, and one thread then
// releases them all at agent scope -- a write-back of this XCD's L2, which
// every store of the workgroup has reached -- before the count.  An
// agent-scope fence per wavefront would write the L2 back eight times.  The
// last workgroup acquires (one invalidation serves the whole workgroup: its
// wavefronts share the compute unit's L1 and the XCD's L2) before anyone
// reads what the others published, and puts the counter back to zero for the
// next call (all n arrivals of this call have happened).  No workgroup waits
// for another.
__device__ __forceinline__ bool arrive_last(int32_t* cnt, int n, int* flag) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const int old = atomicAdd(cnt, 1);
        const bool last = old == n - 1;
        if (last) {
            atomicExch(cnt, 0);
            __threadfence();
        }
        *flag = last ? 1 : 0;
    }
    __syncthreads();
    return *flag != 0;
}

// One tail of the fused epilogue: the wavefront merges rows wave, wave + 8,
// ... of row block rb, each over n parts (key splits or shards) of `In`
// payload.  addr(row, &o0, &lrow) places a row's first part and its LSE,
// store(row, acc, M, S) writes the result.  For n <= 8 four rows are merged
// at once (merge_rows_batch: their loads all in flight together); beyond
// that one row at a time.  The arithmetic is the same either way.
template <typename In, int N, typename Addr, typename Store>
__device__ __forceinline__ void tail_batched(int rb, int rows, int wave, const void* src, int64_t a_ss, int64_t l_ss,
                                             int64_t sc_off, float to_log2, Addr addr, Store store) {
    constexpr int R = 4;
    for (int k0 = 0; k0 < kRowsPerWave; k0 += R) {
        int64_t o0[R];
        const float* lr[R];
        int row[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            row[r] = rb * kMlaRowsPerBlock + wave + kWaves * (k0 + r);
            addr(min(row[r], rows - 1), o0[r], lr[r]);  // rows past the end repeat the last one, unstored
        }
        float acc[R][8], M[R], S[R];
        mrow::merge_rows_batch<R, N, In>(src, o0, a_ss, lr, l_ss, sc_off, to_log2, acc, M, S);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (row[r] < rows) store(row[r], acc[r], M[r], S[r]);
    }
}

template <typename In, typename Addr, typename Store>
__device__ __forceinline__ void tail_rows(int n, int rb, int rows, int wave, const void* src, int64_t a_ss,
                                          int64_t l_ss, int64_t sc_off, float to_log2, Addr addr, Store store) {
    switch (n) {
#define DCP_TAIL_CASE(k) \
    case k: tail_batched<In, k>(rb, rows, wave, src, a_ss, l_ss, sc_off, to_log2, addr, store); return;
        DCP_TAIL_CASE(1)
        DCP_TAIL_CASE(2)
        DCP_TAIL_CASE(3)
        DCP_TAIL_CASE(4)
        DCP_TAIL_CASE(5)
        DCP_TAIL_CASE(6)
        DCP_TAIL_CASE(7)
        DCP_TAIL_CASE(8)
#undef DCP_TAIL_CASE
        default: break;
    }
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int row = rb * kMlaRowsPerBlock + wave + kWaves * k;
        if (row >= rows) break;
        int64_t o0;
        const float* lr;
        addr(row, o0, lr);
        float acc[8], M, S;
        mrow::merge_row_any<8, In>(src, o0, a_ss, lr, l_ss, sc_off, n, to_log2, acc, M, S);
        store(row, acc, M, S);
    }
}

typedef __attribute__((address_space(4))) const MlaArgs KernArgs;

// The fused epilogue (fixed length): once this workgroup's rows are stored,
// (1) with several splits per shard, the last workgroup of (row block, shard)
// to arrive reduces the shard's splits into o_part / lse_part, and (2) the
// last shard of the row block to complete merges the cp shards of every row
// into out / out_lse.  Both reductions are the merge's own row arithmetic
// (merge_row.h), one wavefront per row, so the results equal those of the
// split-reduction launch and of dcp_lse_combine over o_part / lse_part.
template <typename T>
__device__ __forceinline__ void fused_epilogue(const int* work) {
    __shared__ int flag;
    typedef typename T::merge_t Out;
    // The arguments (the kernel's only one, at the start of its argument
    // segment) are read through a pointer the compiler cannot see through,
    // so their loads stay here instead of being hoisted above the key loop
    // and held in registers across it.  The work item comes back from LDS
    // for the same reason.
    KernArgs* ap = (KernArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(ap));
    KernArgs& a = *ap;
    const int rb = __builtin_amdgcn_readfirstlane(work[0]);
    const int s = __builtin_amdgcn_readfirstlane(work[1]);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int hq = a.hq;
    if (a.nsplit > 1) {
        if (!arrive_last(a.split_cnt + rb * a.cp + s, a.nsplit, &flag)) return;
        uint16_t* const o = a.o;
        float* const lse = a.lse;
        const uint16_t* const part_o = a.part_o;
        const float* const part_lse = a.part_lse;
        const int64_t part_sb = a.part_sb, o_sb = a.o_sb, o_sh = a.o_sh, lse_sb = a.lse_sb;
        const float from_log2 = a.from_log2;
        auto addr = [&](int row, int64_t& o0, const float*& lr) {
            const int b = row / hq, h = row - b * hq;
            const int64_t prow = b * part_sb + static_cast<int64_t>(s) * hq + h;  // split 0's partial row
            o0 = prow * kDv + 8 * lane;
            lr = part_lse + prow;
        };
        auto store = [&](int row, const float (&acc)[8], float M, float S) {
            const int b = row / hq, h = row - b * hq;
            const int64_t u = static_cast<int64_t>(s) * hq + h;
            *reinterpret_cast<mrow::u32x4*>(o + b * o_sb + u * o_sh + 8 * lane) = mrow::pack8<Out>(acc);
            if (lane == 0) lse[b * lse_sb + u] = mrow::merged_lse(M, S, from_log2);
        };
        tail_rows<mrow::Payload16<mrow::F16, false, true>>(a.nsplit, rb, a.rows, wave, part_o,
                                                           static_cast<int64_t>(a.cp) * hq * kDv,
                                                           static_cast<int64_t>(a.cp) * hq, a.part_scale - a.part_lse,
                                                           a.to_log2, addr, store);
    }
    if (!arrive_last(a.rb_cnt + rb, a.cp, &flag)) return;
    uint16_t* const out = a.out;
    float* const out_lse = a.out_lse;
    const float* const lse = a.lse;
    const int64_t o_sb = a.o_sb, o_sh = a.o_sh, lse_sb = a.lse_sb, out_sb = a.out_sb, out_sh = a.out_sh,
                  out_lse_sb = a.out_lse_sb;
    const float from_log2 = a.from_log2;
    auto addr = [&](int row, int64_t& o0, const float*& lr) {
        const int b = row / hq, h = row - b * hq;
        o0 = b * o_sb + h * o_sh + 8 * lane;
        lr = lse + b * lse_sb + h;
    };
    auto store = [&](int row, const float (&acc)[8], float M, float S) {
        const int b = row / hq, h = row - b * hq;
        __builtin_nontemporal_store(mrow::pack8<Out>(acc),
                                    reinterpret_cast<mrow::u32x4*>(out + b * out_sb + h * out_sh + 8 * lane));
        if (lane == 0 && out_lse) out_lse[b * out_lse_sb + h] = mrow::merged_lse(M, S, from_log2);
    };
    tail_rows<mrow::Payload16<Out, false>>(a.cp, rb, a.rows, wave, a.o, static_cast<int64_t>(hq) * o_sh, hq, 0,
                                           a.to_log2, addr, store);
}

template <typename T, bool Fused, bool Deep>
__global__ __launch_bounds__(kThreads) void mla_decode_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tiles[3][kTileAlloc];
    __shared__ TileExchange exs[3];
    __shared__ float lsum[kMlaRowsPerBlock];
    __shared__ float amaxp[kWaves][kMlaRowsPerBlock];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;  // query row of this lane within the wavefront
    const int g = lane >> 4;    // lane group: keys 4g..4g+3 of each 16-key half
    // The token(s) and cache of this workgroup.  One shared cache of T rows,
    // row blocks of 128 consecutive (token, head) rows and splits of
    // a.split_len keys; or, with seq_lens, item blockIdx.x of the planning
    // kernel's work list: token b's own cache of min(max(seq_lens[b], 0), T)
    // rows, row blocks that never span tokens, and the plan's split length.
    Work wk;
    int64_t L = a.T;
    int64_t split_len = a.split_len;
    const uint16_t* cache = a.kv;
    int b_tok = 0, h_base = 0;
    if (a.seq_lens) {
        // The item is read before the count is checked: entries past the
        // count are inside the list's capacity (the grid), merely unused.
        const VarlenItem it = a.vl_items[blockIdx.x];
        const int n_items = a.vl_hdr->n_items;
        split_len = a.vl_hdr->split_tiles * kKeys;
        if (static_cast<int>(blockIdx.x) >= n_items) return;
        const int per_token = a.rb_per_token * a.cp;
        b_tok = it.pair / per_token;
        const int rem = it.pair - b_tok * per_token;
        const int rbi = rem / a.cp;
        wk.rb = b_tok * a.rb_per_token + rbi;
        wk.s = rem - rbi * a.cp;
        wk.p = it.p;
        wk.slot = it.slot;
        h_base = rbi * kMlaRowsPerBlock;
        L = min(max(static_cast<int64_t>(a.seq_lens[b_tok]), int64_t{0}), a.T);
        cache = a.kv + b_tok * a.kv_sb;
    } else {
        wk = work_of(a);
    }
    __shared__ int fused_work[2];  // (row block, shard) for the fused epilogue
    if (Fused && tid == 0) {
        fused_work[0] = wk.rb;
        fused_work[1] = wk.s;
    }
    // Shard s: n_s logical keys, key j at cache row start + j * step.
    int64_t start, n_s;
    int step;
    if (a.interleaved) {
        start = wk.s;
        step = a.cp;
        n_s = L > wk.s ? (L - wk.s + a.cp - 1) / a.cp : 0;
    } else {
        start = (static_cast<int64_t>(wk.s) * L) / a.cp;
        step = 1;
        n_s = (static_cast<int64_t>(wk.s + 1) * L) / a.cp - start;
    }
    const KeyRows kr{cache + start * a.kv_st, static_cast<int32_t>(step * a.kv_st)};
    // Logical key range of this split.
    const int64_t k0 = static_cast<int64_t>(wk.p) * split_len;
    const int64_t k1 = min(k0 + split_len, n_s);
    const int ntiles = k0 < k1 ? static_cast<int>((k1 - k0 + kKeys - 1) / kKeys) : 0;
    // Every tile but a split's last is full and takes the scalar-address copy.
    const bool full_ok = kr.rstride < kFullTileMaxStride;
    const uint32_t lane_off = full_tile_lane_offset(kr.rstride, wave, lane);
    auto copy_tile = [&](int j, uint16_t* dst) {
        if (full_ok && j + 1 < ntiles)
            dma_tile_full(kr, dst, k0 + static_cast<int64_t>(j) * kKeys, lane_off, wave);
        else
            dma_tile(kr, dst, k0 + static_cast<int64_t>(j) * kKeys, k1, wave, lane);
    };
    if (ntiles > 0) copy_tile(0, tiles[0]);

    // Q fragments: fragment f holds columns 32f + 8g .. +7 of this lane's
    // query row, row 16 wave + r16 of the workgroup (rows past the end repeat
    // the last row and are not stored).  In that layout each 16-lane pass of a
    // load instruction would read 16 rows, 16 B apiece: 16 cache lines.  The
    // vector memory unit serves a 16-byte load at about one cache line per
    // clock and pass (measured on L2-resident data: 18 B per clock and
    // compute unit for 16 rows x 16 B per pass, 53 for 4 rows x 64 B, 127 for
    // 256 contiguous bytes).  So lane 4R + c loads columns 32f + 8c .. of row
    // R (each pass: 4 rows x 64 B), and a lane permutation (ds_bpermute, no
    // LDS storage) hands lane 16g + r16 the words of lane 4 r16 + g.
    const RowPlace rp{wk.rb, b_tok, h_base, a.seq_lens != nullptr};
    typename T::v8 qf[kQSteps];
    {
        int bq, hq;
        bool vq;
        place_row(a, rp, kRowsPerWave * wave + (lane >> 2), bq, hq, vq);
        const uint16_t* qsrc = a.q + bq * a.q_sb + hq * a.q_sh + 8 * (lane & 3);
#pragma unroll
        for (int f = 0; f < kQSteps; ++f) qf[f] = as_v8<T>(*reinterpret_cast<const u32x4*>(qsrc + 32 * f));
        // Settle these loads (and tile 0's copies) here: a wait for them left
        // inside the key loop would also wait for the tile copies in flight there.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        const int src = 4 * (4 * r16 + g);  // byte address of the source lane
#pragma unroll
        for (int f = 0; f < kQSteps; ++f) {
            u32x4 w = __builtin_bit_cast(u32x4, qf[f]);
#pragma unroll
            for (int d = 0; d < 4; ++d) w[d] = __builtin_amdgcn_ds_bpermute(src, w[d]);
            qf[f] = as_v8<T>(w);
        }
    }

    // Operand offsets.  q.k step f: key r16, chunk 4f + g, in block f at slot
    // 16 g + (r16 ^ 8 (f % 2)).  p.v tile t = 4j + u: key k = 4g + r16/4 and
    // quarter qq = r16 % 4 of the tile's 16 columns: chunk c = 8j + u (qq < 2)
    // or c + 4 (qq >= 2), i.e. block 2j + qq/2 at slot 16u + (k ^ 8 (qq/2)),
    // plus 4 elements for the odd quarters.
    LaneOffsets off;
    {
        off.s_even = 8 * (16 * g + r16);
        off.s_odd = 8 * (16 * g + (r16 ^ 8));
        const int key = 4 * g + (r16 >> 2);
        const int qh = (r16 & 3) >> 1;
        const int tr0 = kBlockElems * qh + 8 * (key ^ (8 * qh)) + 4 * (r16 & 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) off.tr[u] = tr0 + 128 * u;
    }

    f32x4 acc[kWaves][4];
#pragma unroll
    for (int rt = 0; rt < kWaves; ++rt)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of row r16, log2 units
    float l_run = 0.0f;       // lane-partial running sum of row r16

    if constexpr (Deep) {
        // Two tiles in flight: tile i lives in buffer i % 3 and runs its
        // scores and its p.v in one interval, with a barrier between them (the
        // p.v needs every wavefront's P^T); the copies of tiles i + 1 and
        // i + 2 are in flight meanwhile, so each has two intervals to land.
        // For workgroups whose key range no other workgroup reads (one row
        // block), where every tile comes from HBM rather than the L2.
        // Every tile copy is four (wavefronts 4-7) or five (0-3) loads, and
        // nothing else in the loop touches vector memory, so vmcnt(4) leaves
        // at most the newest copy's loads in flight: the older tile is in.
        static_assert(kDmaPerTile / kWaves >= 4, "vmcnt(4) needs at least four copies per wavefront and tile");
        if (ntiles > 1) copy_tile(1, tiles[1]);
        int cur = 0;
        // Every tile but the last: its copy and the next one's were issued
        // two intervals and one interval ago.
        for (int it = 0; it + 1 < ntiles; ++it) {
            if (it > 0) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): tile it is in, it + 1 may not be
            __syncthreads();  // tile it visible; tile it - 1's buffer and the exchange are free
            const int far = cur == 0 ? 2 : cur - 1;
            if (it + 2 < ntiles) copy_tile(it + 2, tiles[far]);
            qk_tile<T, false>(a, tiles[cur], off, qf, m_run, l_run, k0 + static_cast<int64_t>(it) * kKeys, k1, g,
                              wave, lane, exs[0]);
            __syncthreads();
            pv_tile<T>(tiles[cur], off, acc, exs[0], wave, lane);
            cur = cur == 2 ? 0 : cur + 1;
        }
        // The last tile, with the key mask.
        if (ntiles > 0) {
            if (ntiles > 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            qk_tile<T, true>(a, tiles[cur], off, qf, m_run, l_run, k0 + static_cast<int64_t>(ntiles - 1) * kKeys, k1,
                             g, wave, lane, exs[0]);
            __syncthreads();
            pv_tile<T>(tiles[cur], off, acc, exs[0], wave, lane);
        }
    } else {
        // Tile i lives in buffer i % 3 with exchange i % 3.  Its scores and
        // softmax run one interval before its p.v: between barriers i and i + 1
        // every wavefront runs p.v of tile i (which needs every wavefront's P^T
        // of tile i, published before barrier i) and the scores of tile i + 1.
        // A buffer is therefore busy for two intervals, and the copy of tile
        // i + 2, issued after barrier i into the buffer tile i - 1 left, has one
        // interval to land (barrier i + 1 waits for it).
        if (ntiles > 1) copy_tile(1, tiles[1]);
        __syncthreads();  // tile 0: every wavefront waited for its own copies above
        if (ntiles > 0) qk_tile<T, true>(a, tiles[0], off, qf, m_run, l_run, k0, k1, g, wave, lane, exs[0]);
        // A rolled loop: the buffer and exchange indices are wave-uniform, so
        // the LDS addresses are formed per tile instead of being held in
        // registers for every buffer (unrolled by three, the loop spills).  The
        // last tile's p.v runs after the loop, so that inside it p.v and the
        // next scores form one block of straight-line code.
        // Tiles 1 .. ntiles - 2 are full; only the last one's scores need the
        // key mask, so its interval runs after the loop.
        int cur = 0;
        for (int it = 0; it + 2 < ntiles; ++it) {
            const int64_t t0 = k0 + static_cast<int64_t>(it) * kKeys;
            const int nxt = cur == 2 ? 0 : cur + 1;
            const int prv = cur == 0 ? 2 : cur - 1;
            all_tiles_ready();
            // Each copy holds the vector memory unit for about 64 clocks (16
            // keys x 64 B: 16 cache lines per 16-lane pass), ~2300 per tile
            // and workgroup; a wavefront issuing all of its copies at once
            // waits at the issue behind the other wavefronts' copies.  Three
            // go out before p.v and the rest after it (measured: 1-1.5%
            // faster than all five before, 3.5% faster than all after).
            const bool split_copy = full_ok && it + 3 < ntiles;  // tile it + 2 is full
            const int64_t tc = k0 + static_cast<int64_t>(it + 2) * kKeys;
            if (split_copy)
                dma_tile_full<0, 3>(kr, tiles[prv], tc, lane_off, wave);
            else
                copy_tile(it + 2, tiles[prv]);
            pv_tile<T>(tiles[cur], off, acc, exs[cur], wave, lane);
            if (split_copy) dma_tile_full<3>(kr, tiles[prv], tc, lane_off, wave);
            qk_tile<T, false>(a, tiles[nxt], off, qf, m_run, l_run, t0 + kKeys, k1, g, wave, lane, exs[nxt]);
            cur = nxt;
        }
        if (ntiles > 1) {
            const int nxt = cur == 2 ? 0 : cur + 1;
            all_tiles_ready();
            pv_tile<T>(tiles[cur], off, acc, exs[cur], wave, lane);
            qk_tile<T, true>(a, tiles[nxt], off, qf, m_run, l_run, k0 + static_cast<int64_t>(ntiles - 1) * kKeys, k1, g,
                             wave, lane, exs[nxt]);
            cur = nxt;
        }
        if (ntiles > 0) {
            all_tiles_ready();
            pv_tile<T>(tiles[cur], off, acc, exs[cur], wave, lane);
        }
    }

    const bool direct = a.seq_lens ? wk.slot < 0 : a.nsplit == 1;
    store_block<T>(a, wk, rp, wave, lane, acc, m_run, l_run, direct, lsum, amaxp);
    if (Fused) fused_epilogue<T>(fused_work);
}

}  // namespace
}  // namespace dcp

namespace dcp {

// Enqueue a validated plan: the decode kernel, then (several splits) the
// merge over splits.
int run_mla(const MlaPlan& plan, void* hip_stream, const char* fn) {
    if (plan.blocks == 0) return ok();
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const dim3 grid(static_cast<unsigned>(plan.blocks));
    if (plan.varlen) {
        const hipError_t e = static_cast<hipError_t>(varlen_plan_launch(plan.args, stream));
        if (e != hipSuccess) return fail(DCP_ERR_HIP, "%s: launch of the planning kernel failed: %s", fn,
                                         hipGetErrorString(e));
    }
    const bool f16 = plan.args.dtype == DCP_DTYPE_FP16;
    if (plan.args.fused) {
        if (f16)
            mla_decode_kernel<F16, true, false><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
        else
            mla_decode_kernel<Bf16, true, false><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
    } else if (plan.deep) {
        if (f16)
            mla_decode_kernel<F16, false, true><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
        else
            mla_decode_kernel<Bf16, false, true><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
    } else if (f16) {
        mla_decode_kernel<F16, false, false><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
    } else {
        mla_decode_kernel<Bf16, false, false><<<grid, dim3(kThreads), 0, stream>>>(plan.args);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && plan.varlen) {
        if (plan.args.slots > 0) e = static_cast<hipError_t>(varlen_reduce_launch(plan.args, stream));
    } else if (e == hipSuccess && plan.args.nsplit > 1 && !plan.args.fused) {
        // The splits of every (token, shard, head) are merged like DCP shards;
        // with reduce_merge the same launch also merges each head's shards.
        if (plan.reduce_merge)
            e = static_cast<hipError_t>(
                reduce_merge_launch(plan.reduce, plan.shard_merge, plan.B, plan.args.hq, stream));
        else
            e = static_cast<hipError_t>(merge_launch_all(plan.reduce, plan.B, stream));
    }
    if (e == hipSuccess && plan.merge_shards && !plan.reduce_merge)
        e = static_cast<hipError_t>(merge_launch_all(plan.shard_merge, plan.B, stream));
    if (e != hipSuccess) return fail(DCP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace dcp

extern "C" int dcp_mla_partial_decode(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                                      int64_t kv_tokens, int64_t kv_st, int dtype, int cp, float softmax_scale,
                                      int lse_mode, void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part,
                                      int64_t lse_sb, void* scratch, size_t scratch_bytes, void* hip_stream) {
    dcp::MlaPlan plan;
    const int rc = dcp::plan_mla(q, B, hq, q_sb, q_sh, kv, kv_tokens, kv_st, nullptr, dtype, cp, softmax_scale,
                                 lse_mode, o_part, o_sb, o_sh, lse_part, lse_sb, scratch, scratch_bytes, &plan);
    if (rc != DCP_OK) return rc;
    return dcp::run_mla(plan, hip_stream, "dcp_mla_partial_decode");
}

extern "C" int dcp_mla_partial_decode_varlen(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh,
                                             const void* kv, int64_t kv_sb, int64_t kv_st, int64_t max_seq_len,
                                             const int32_t* seq_lens, int kv_layout, int dtype, int cp,
                                             float softmax_scale, int lse_mode, void* o_part, int64_t o_sb,
                                             int64_t o_sh, float* lse_part, int64_t lse_sb, void* scratch,
                                             size_t scratch_bytes, void* hip_stream) {
    dcp::MlaPlan plan;
    const dcp::MlaVarlen vl{seq_lens, kv_sb, kv_layout};
    const int rc = dcp::plan_mla(q, B, hq, q_sb, q_sh, kv, max_seq_len, kv_st, &vl, dtype, cp, softmax_scale,
                                 lse_mode, o_part, o_sb, o_sh, lse_part, lse_sb, scratch, scratch_bytes, &plan);
    if (rc != DCP_OK) return rc;
    return dcp::run_mla(plan, hip_stream, "dcp_mla_partial_decode_varlen");
}

extern "C" int dcp_mla_decode_merged(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                                     int64_t kv_tokens, int64_t kv_st, int dtype, int cp, float softmax_scale,
                                     int lse_mode, void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part,
                                     int64_t lse_sb, void* out, int64_t out_sb, int64_t out_sh, float* out_lse,
                                     int64_t out_lse_sb, int fuse, void* scratch, size_t scratch_bytes,
                                     void* hip_stream) {
    dcp::MlaPlan plan;
    const int rc = dcp::plan_mla_merged(q, B, hq, q_sb, q_sh, kv, kv_tokens, kv_st, dtype, cp, softmax_scale,
                                        lse_mode, o_part, o_sb, o_sh, lse_part, lse_sb, out, out_sb, out_sh, out_lse,
                                        out_lse_sb, fuse, scratch, scratch_bytes, &plan);
    if (rc != DCP_OK) return rc;
    return dcp::run_mla(plan, hip_stream, "dcp_mla_decode_merged");
}
