// merge_row.h -- the per-row arithmetic of the DCP LSE merge, in one place.
//
// Every kernel that merges LSE-weighted partials -- the merge of DCP shards
// (merge.hip), the reduction of the MLA decode's key splits (the same merge
// kernel over scratch partials, the variable-length reducer in mla_varlen.hip,
// and the fused epilogue of mla_decode.hip) -- forms one row's result with the
// functions below, so they all give the same bits for the same inputs:
//     M = max over s (exact in any order);   w_s = 2^((lse_s - M) * c), 0 for lse_s = -inf;
//     S = sum of w_s: for n <= 16 ascending from 0; for n > 16 per group of
//         64 shards a fixed tree (tree_sum), the groups' sums added in
//         ascending order from 0;   inv = 1/S (0 when S = 0);
//     w^_s = w_s * inv (* the row's scale factor, for scaled partials);
//     acc = sum of w^_s * O_s in fp32 FMAs, a shard of weight 0 adding +0:
//         for n <= 16 ascending from 0; for n > 16 per group of 16 shards
//         (16q .. 16q+15) ascending from 0, the groups' sums then added in
//         ascending order (so the groups of a row can run in parallel);
//     L = M + log2(S) / c.
// ("[DCP] Run fi_a2a on FlashInfer's fused all-to-all + LSE reduce", sglang PR
// #40539, Motivation; "[Attention] Add direct symmetric-memory DCP A2A", vLLM
// PR #48897: weights formed in fp32, empty shards publish -inf and their
// payload is skipped.)  c = 1 for base-2 LSEs and log2 e for natural ones.
// A lane owns 8 consecutive columns of the row: one 16-byte load per shard.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace dcp {
namespace mrow {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The two 16-bit payload types.  A 32-bit word holds two elements, the
// lower-addressed one in the low half; widening to fp32 is exact for both,
// narrowing rounds to nearest even.
struct Bf16 {
    static constexpr bool kFoldsIntoFma = false;
    // bf16 is the high half of an fp32: shifting or masking widens it.
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
    }
};

struct F16 {
    // The compiler may fold the last FMA of a sum and its conversion to fp16
    // into one mixed-precision FMA that rounds once; pack8 keeps the two
    // roundings the arithmetic states (fp32, then fp16) on every path.
    static constexpr bool kFoldsIntoFma = true;
    static __device__ __forceinline__ float lo(uint32_t w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(a))) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(b))) << 16);
    }
};

// One 16-byte load, non-temporal (NT) or plain.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

// How a lane reads its 8 columns of one shard row and accumulates them.
// Scaled: the row was stored multiplied by a power of two (the MLA decode's
// split partials, fp16, inside the library only); its weight is multiplied
// by the factor stored sc_off floats after its LSE.  zero_unless replaces the
// row by zeros -- a select on the loaded words, not a branch, so the loads
// stay ahead of their use -- and the all-zero word is +0 in every payload
// type, so an empty shard adds exactly +0 whatever it held (NaN included).
template <typename T, bool NT, bool Scaled = false>
struct Payload16 {
    static constexpr bool kScaled = Scaled;
    typedef u32x4 row_t;
    static __device__ __forceinline__ row_t load(const void* base, int64_t off) {
        return load16<NT>(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off));
    }
    static __device__ __forceinline__ row_t zero_unless(bool use, row_t v) {
        row_t z;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = use ? v[i] : 0u;
        return z;
    }
    static __device__ __forceinline__ void fma(float (&acc)[8], float w, row_t v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, T::lo(v[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, T::hi(v[i]), acc[2 * i + 1]);
        }
    }
};

// acc += w * v; a shard with weight exactly 0 (an empty one) adds +0.  For a
// nonzero w this is In::fma(acc, w, v) exactly.
template <typename In>
__device__ __forceinline__ void fma8(float (&acc)[8], float w, typename In::row_t v) {
    In::fma(acc, w, In::zero_unless(w != 0.0f, v));
}

// Unnormalised weight of a shard with LSE x against the row maximum M.
// v_exp_f32 is the hardware's 1-ulp exp2; an exponent below -126 flushes
// the weight to 0, i.e. a shard under 2^-126 of the largest is skipped.
__device__ __forceinline__ float shard_weight(float x, float M, float to_log2) {
    return (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((x - M) * to_log2);
}

// 1/S, or 0 when every shard is empty (S = 0).
__device__ __forceinline__ float inv_sum(float S) { return (S > 0.0f) ? __builtin_amdgcn_rcpf(S) : 0.0f; }

// The merged LSE in the input's base; S = 0 (all shards empty, M = -inf)
// gives -inf.
__device__ __forceinline__ float merged_lse(float M, float S, float from_log2) {
    return M + __builtin_amdgcn_logf(S) * from_log2;
}

// The lane's 8 accumulators rounded to the output type, as one 16-byte word.
// For fp16 the fp32 sums pass through an empty asm first, so the conversion
// cannot be merged with the FMA that produced them.
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float (&acc_in)[8]) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[i] = acc_in[i];
        if (T::kFoldsIntoFma) asm volatile("" : "+v"(acc[i]));
    }
    u32x4 p;
    p[0] = T::pack(acc[0], acc[1]);
    p[1] = T::pack(acc[2], acc[3]);
    p[2] = T::pack(acc[4], acc[5]);
    p[3] = T::pack(acc[6], acc[7]);
    return p;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], then
// row_half_mirror and row_mirror.  Applied in that order they combine all 16
// lanes of a row, and every lane of the row ends up holding the result.
template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// Maximum over the first m <= 64 lanes (lanes >= m must hold -inf), in a
// scalar register.  fmaxf is exact, so any order gives the same value.
__device__ __forceinline__ float wave_max(float v, int m) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    float r = lane_value(v, 0);
    if (m > 16) r = fmaxf(r, lane_value(v, 16));
    if (m > 32) r = fmaxf(fmaxf(r, lane_value(v, 32)), lane_value(v, 48));
    return r;
}

// Sum over the first m <= 64 lanes (lanes >= m must hold 0) in one fixed
// order: within each 16-lane row the DPP tree (pairs, quads, halves, rows),
// then row 0 + row 1, plus (row 2 + row 3).  Every path that merges more than
// 16 parts sums them this way, so they agree bit for bit.
__device__ __forceinline__ float tree_sum(float v, int m) {
    v = v + dpp<0xB1>(v);
    v = v + dpp<0x4E>(v);
    v = v + dpp<0x141>(v);
    v = v + dpp<0x140>(v);
    float r = lane_value(v, 0);
    if (m > 16) r = r + lane_value(v, 16);
    if (m > 32) r = r + (lane_value(v, 32) + lane_value(v, 48));
    return r;
}

// M and S of m <= 64 parts held one per lane (x: the lane's LSE, -inf in
// lanes >= m), by the rules above.  All 64 lanes, wave-uniform m.
__device__ __forceinline__ void lane_max_sum(float x, int m, float to_log2, float& M, float& S) {
    M = wave_max(x, m);
    const float w = shard_weight(x, M, to_log2);
    if (m <= 16) {
        S = 0.0f;
        for (int i = 0; i < m; ++i) S += lane_value(w, i);
    } else {
        S = 0.0f + tree_sum(w, m);
    }
}

// The lane's LSE of part c0 + lane of a row (-inf past the m-th).
__device__ __forceinline__ float lane_lse(const float* lrow, int64_t l_ss, int c0, int m) {
    const int lane = threadIdx.x & 63;
    return lane < m ? lrow[static_cast<int64_t>(c0 + lane) * l_ss] : -INFINITY;
}

// M and S of a row of n > 64 parts whose LSEs are lrow[s * l_ss], 64 at a
// time (all 64 lanes, wave-uniform arguments).
__device__ __forceinline__ void row_max_sum(const float* lrow, int64_t l_ss, int n, float to_log2, float& M,
                                            float& S) {
    M = 0.0f;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const float cm = wave_max(lane_lse(lrow, l_ss, c0, min(64, n - c0)), min(64, n - c0));
        M = c0 == 0 ? cm : fmaxf(M, cm);
    }
    S = 0.0f;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int m = min(64, n - c0);
        S += tree_sum(shard_weight(lane_lse(lrow, l_ss, c0, m), M, to_log2), m);
    }
}

// Merge of one row over a runtime number n >= 1 of shards, called by all 64
// lanes of a wavefront with wave-uniform arguments.  Shard s's 8 columns of
// this lane are In elements at attn + o0 + s*a_ss (o0 includes the lane's
// column offset); its LSE is lrow[s*l_ss] and, for scaled payloads, its
// factor lrow[s*l_ss + sc_off].  The LSEs come in 64 at a time, shard c0 + l
// in lane l, for the maximum and the sum (lane_max_sum, row_max_sum); the
// payloads come G shards at a time (G divides kAccGroup), the next group's
// loads issued before the current group's FMAs.  Returns the accumulators, M
// and S.
constexpr int kAccGroup = 16;  // shards per group of the accumulation
template <int G, typename In>
__device__ __forceinline__ void merge_row_any(const void* attn, int64_t o0, int64_t a_ss, const float* lrow,
                                              int64_t l_ss, int64_t sc_off, int n, float to_log2, float (&acc)[8],
                                              float& M, float& S) {
    const int lane = threadIdx.x & 63;
    typedef typename In::row_t row_t;
    // The first 64 parts' LSEs (and factors) are read once, with the first
    // payload loads, so that only one memory round trip precedes the weights.
    const int m0 = min(64, n);
    const float x0 = lane_lse(lrow, l_ss, 0, m0);
    const float sc0 = In::kScaled && lane < m0 ? lrow[static_cast<int64_t>(lane) * l_ss + sc_off] : 0.0f;
    row_t cur[G], nxt[G];
#pragma unroll
    for (int i = 0; i < G; ++i) cur[i] = In::load(attn, o0 + static_cast<int64_t>(min(i, n - 1)) * a_ss);

    if (n <= 64) {
        lane_max_sum(x0, n, to_log2, M, S);
    } else {
        row_max_sum(lrow, l_ss, n, to_log2, M, S);
    }
    const float inv = inv_sum(S);

    static_assert(kAccGroup % G == 0 && 64 % kAccGroup == 0, "load groups tile the accumulation groups");
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;  // n = 0; otherwise the first group's sum replaces it
    float grp[8];  // the current accumulation group's sum
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int m = min(64, n - c0);
        float wl = shard_weight(c0 == 0 ? x0 : lane_lse(lrow, l_ss, c0, m), M, to_log2) * inv;
        if (In::kScaled)
            wl *= c0 == 0 ? sc0 : (lane < m ? lrow[static_cast<int64_t>(c0 + lane) * l_ss + sc_off] : 0.0f);
        for (int g0 = 0; g0 < m; g0 += G) {
            const int s0 = c0 + g0;     // first shard of this load group
            const int s_next = s0 + G;  // first shard of the next one
            if (s_next < n) {
#pragma unroll
                for (int i = 0; i < G; ++i)
                    nxt[i] = In::load(attn, o0 + static_cast<int64_t>(min(s_next + i, n - 1)) * a_ss);
            }
            if (s0 % kAccGroup == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) grp[i] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < G; ++i)
                if (g0 + i < m) fma8<In>(grp, lane_value(wl, g0 + i), cur[i]);
            if (s_next % kAccGroup == 0 || s_next >= n) {  // the accumulation group is complete
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = s0 < kAccGroup ? grp[i] : acc[i] + grp[i];
            }
            if (s_next < n) {
#pragma unroll
                for (int i = 0; i < G; ++i) cur[i] = nxt[i];
            }
        }
    }
}

// R rows of N shards each (N known at compile time), all R * N payload loads
// issued before any arithmetic: for a wavefront that merges several rows in
// turn, the rows' memory latencies overlap instead of adding up.  Row r's
// shard s is at attn + o0[r] + s*a_ss and its LSE at lrow[r][s*l_ss] (wave-
// uniform).  The arithmetic of each row is merge_row_any's, step for step.
template <int R, int N, typename In>
__device__ __forceinline__ void merge_rows_batch(const void* attn, const int64_t (&o0)[R], int64_t a_ss,
                                                 const float* const (&lrow)[R], int64_t l_ss, int64_t sc_off,
                                                 float to_log2, float (&acc)[R][8], float (&M)[R], float (&S)[R]) {
    typename In::row_t v[R][N];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int s = 0; s < N; ++s) v[r][s] = In::load(attn, o0[r] + static_cast<int64_t>(s) * a_ss);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float x[N];
#pragma unroll
        for (int s = 0; s < N; ++s) x[s] = lrow[r][static_cast<int64_t>(s) * l_ss];
        float m = x[0];
#pragma unroll
        for (int s = 1; s < N; ++s) m = fmaxf(m, x[s]);
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < N; ++s) sum += shard_weight(x[s], m, to_log2);
        const float inv = inv_sum(sum);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < N; ++s) {
            float w = shard_weight(x[s], m, to_log2) * inv;
            if (In::kScaled) w *= lrow[r][static_cast<int64_t>(s) * l_ss + sc_off];
            fma8<In>(acc[r], w, v[r][s]);
        }
        M[r] = m;
        S[r] = sum;
    }
}

}  // namespace mrow
}  // namespace dcp
