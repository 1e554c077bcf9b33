/*
 * dcp.h -- C ABI of the MI355X (gfx950) decode-context-parallel LSE merge.
 *
 * Decode context parallelism (DCP) splits the latent KV cache of an MLA model
 * over cp shards.  Each shard runs decode attention for every head over its
 * own tokens and yields a partial output O_s and a log-sum-exp lse_s per
 * (token, head).  The exact attention output is the LSE-weighted merge of the
 * shards' partials ("[DCP] Run fi_a2a on FlashInfer's fused all-to-all + LSE
 * reduce", sglang PR #40539, Motivation; "[Attention] Add direct
 * symmetric-memory DCP A2A", vLLM PR #48897, commit message: the merge
 * weights are formed in fp32):
 *
 *     M = max_s lse_s,  w_s = base^(lse_s - M),  S = sum_s w_s
 *     out = sum_s (w_s / S) O_s,                 L = M + log_base S
 *
 * On one GPU the cp shards are resident buffers: the caller's [B, H, D]
 * attention output is read in place as a [B, H/cp, cp, D] view, head h
 * belonging to shard h / (H/cp) (PR #40539, Modifications).
 *
 * Conventions for every entry point:
 *  - All pointers to tensors are DEVICE pointers owned by the caller; the
 *    library never allocates, frees, synchronises or prints, so every call may
 *    be captured into a HIP graph.  Host-side objects (a workspace) are the
 *    only memory the library allocates, and only in dcp_workspace_create;
 *    device buffers (a workspace's, a producer's scratch) are the caller's.
 *  - Sizes and strides are in ELEMENTS, not bytes.  The innermost (D) stride
 *    of every tensor is 1.
 *  - Every argument is checked before anything is enqueued: on any error the
 *    call returns a nonzero status, nothing has been launched, and
 *    dcp_last_error() (thread-local) names what to change.
 *  - hip_stream is a hipStream_t passed as void*; NULL is the null stream.
 *  - D (the head dimension, the MLA kv_lora_rank) is 512; payloads are bf16
 *    or fp16 (the merge: the workspace's dtype; the MLA decode: its dtype
 *    argument); every LSE is fp32.
 */
#ifndef DCP_H
#define DCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define DCP_OK 0
#define DCP_ERR_INVALID_ARG 1 /* bad size, null pointer, H % cp != 0, out aliases an input      */
#define DCP_ERR_LAYOUT 2      /* unsupported D or dtype, negative or overlapping strides         */
#define DCP_ERR_ALIGN 3       /* a pointer or row stride breaks the 16-byte alignment rule      */
#define DCP_ERR_STREAM 4      /* called on a stream other than the workspace's                  */
#define DCP_ERR_WORKSPACE 5   /* no workspace, other geometry, or a device buffer too small        */
#define DCP_ERR_HIP 6         /* the HIP runtime refused a launch                               */

/* LSE base: the attention backend decides which one its LSE is in
 * (PR #40539, Modifications: lse_mode comes from the backend). */
#define DCP_LSE_BASE_E 0 /* lse = ln  sum exp(z)             */
#define DCP_LSE_BASE_2 1 /* lse = log2 sum 2^(z * log2 e)    */

/* LSE layouts (PR #40539, Modifications and Accuracy Tests). */
#define DCP_LSE_BHC 0 /* [B, H/cp, cp]: element (b, j, s) at b*l0 + j*l1 + s*l2              */
#define DCP_LSE_BH1 1 /* FlashMLA [B, H, 1]: element (b, h) at b*l0 + h*l1, h = s*(H/cp) + j */

/* Element types of the merge payload (attn and out). */
#define DCP_DTYPE_BF16 0
#define DCP_DTYPE_FP16 1 /* IEEE binary16 */

#define DCP_HEAD_DIM 512 /* value / merged head dimension (the MLA kv_lora_rank)   */
#define DCP_QK_DIM 576   /* query/key columns of the MLA decode: 512 latent + 64 rope */
#define DCP_MAX_CP 64

/* How dcp_lse_combine reads its partials and writes its output
 * (dcp_workspace_set_load_policy). */
#define DCP_LOAD_STREAMING 0 /* non-temporal: partials read from HBM once (default) */
#define DCP_LOAD_CACHED 1    /* plain loads: partials just written and still cache-resident */

/* Which cache rows a DCP shard owns (dcp_mla_partial_decode_varlen). */
#define DCP_KV_CONTIGUOUS 0  /* shard s: rows [floor(s*L/cp), floor((s+1)*L/cp)) of a length-L cache */
#define DCP_KV_INTERLEAVED 1 /* shard s: rows t < L with t mod cp == s                              */

typedef struct dcp_workspace dcp_workspace;

/*
 * Bytes of device memory a merge workspace needs (dcp_workspace_create's
 * dev_buf): its receive-buffer landing zone for up to capacity_tokens tokens,
 * i.e. capacity_tokens * h_local * cp rows of d payload elements plus one fp32
 * LSE per row, each region rounded up to 256 bytes.  The pages size their
 * fused-reduce workspaces with such a function, by the widest decode batch
 * times the local heads ("[DCP] Run fi_a2a on FlashInfer's fused all-to-all +
 * LSE reduce", sglang PR #40539, Coordination, and Speed Tests and Profiling,
 * memory), from the geometry a caller holds at initialisation (maximum
 * tokens, heads per rank, head dimension, dtype: "[Attention] Add direct
 * symmetric-memory DCP A2A", vLLM PR #48897, review thread).  Arguments and
 * errors as dcp_workspace_create; *bytes receives the size.
 */
int dcp_workspace_size(int64_t capacity_tokens, int h_local, int cp, int d, int dtype, size_t* bytes);

/*
 * Create a merge workspace over a caller-owned device buffer.  It fixes the
 * geometry (h_local = H/cp local heads, cp shards, head dimension d, dtype),
 * the token capacity and the ONE stream it serves, as the pages' workspaces
 * do: one per ordered stream, sized by the widest decode batch and created
 * once, before graph capture (PR #40539, Modifications).
 *
 * dev_buf, bytes   device buffer of at least dcp_workspace_size() bytes,
 *                  16-byte aligned, owned by the caller (allocate it with
 *                  PyTorch or hipMalloc; it must outlive the workspace).  It is
 *                  the landing zone: dcp_workspace_recv says where a caller may
 *                  stage the shard partials of up to capacity_tokens tokens to
 *                  merge them with dcp_lse_combine.  The library never reads
 *                  or writes it by itself.  NULL or too small gives
 *                  DCP_ERR_WORKSPACE, misaligned DCP_ERR_ALIGN.
 * capacity_tokens  >= 1; dcp_lse_combine splits wider batches into ordered
 *                  chunks of at most this many tokens (PR #40539,
 *                  Modifications and Coordination).
 * h_local, cp      >= 1; cp <= DCP_MAX_CP.
 * d                DCP_HEAD_DIM.
 * dtype            DCP_DTYPE_BF16 or DCP_DTYPE_FP16: the element type of the
 *                  attn and out buffers of every call on this workspace (the
 *                  pages' merge kernels take fp16 and bf16 payloads, PR #40539
 *                  Motivation; vLLM PR #48897, port commit).
 * hip_stream       the stream every dcp_lse_combine call on this workspace
 *                  must use (opaque value, compared, never dereferenced).
 * ws               receives the handle; release it with dcp_workspace_destroy.
 *
 * On one GPU the shards' partials are usually the caller's resident attention
 * output, which dcp_lse_combine reads in place; the landing zone serves a
 * caller that gathers them first (as an exchange would).
 */
int dcp_workspace_create(void* dev_buf, size_t bytes, int64_t capacity_tokens, int h_local, int cp, int d, int dtype,
                         void* hip_stream, dcp_workspace** ws);

/*
 * The landing zone of ws: shard s of local head j of token b (b < capacity)
 * goes to attn + b*attn_sb + (s*h_local + j)*attn_sh, D elements of the
 * workspace's dtype, and its LSE to lse[b*lse_sb + s*h_local + j], so that
 *     dcp_lse_combine(ws, attn, B, cp*h_local, attn_sb, attn_sh, lse,
 *                     DCP_LSE_BH1, lse_sb, 1, 0, ...)
 * merges the first B staged tokens (head h of the [B, H, D] view belongs to
 * shard h / h_local, PR #40539, Modifications).  attn_sh = D, attn_sb = H*D,
 * lse_sb = H.  Pointers are device pointers inside dev_buf.
 */
int dcp_workspace_recv(const dcp_workspace* ws, void** attn, int64_t* attn_sb, int64_t* attn_sh, float** lse,
                       int64_t* lse_sb);

/* Release a workspace (its host object; the device buffer stays the caller's).  NULL is accepted. */
int dcp_workspace_destroy(dcp_workspace* ws);

/*
 * Cache policy of every later dcp_lse_combine call on ws: how the partials are
 * read.  DCP_LOAD_STREAMING (the default) reads them with non-temporal loads,
 * which do not displace cached data: fastest when the partials come from HBM.
 * DCP_LOAD_CACHED reads them with plain loads: fastest when they were written
 * just before (the exchange's receive buffers, or a producer in the same
 * stream) and still sit in the L2 / Infinity Cache.  The output is written
 * with non-temporal stores under both (measured faster in both cases).
 * Results are bit-identical under both policies.  Returns DCP_ERR_INVALID_ARG for an
 * unknown policy or handle.
 */
int dcp_workspace_set_load_policy(dcp_workspace* ws, int policy);

/*
 * LSE-weighted merge of cp shard partials, read in place.
 *
 * attn      [B, H, D] attention output in the workspace's dtype (bf16 or
 *           fp16), H = cp * h_local of ws.  Token b,
 *           head h, column d at attn + b*attn_sb + h*attn_sh + d.  Shard s of
 *           local head j is head s*h_local + j.  Padded token strides and
 *           heads taken from a wider backing buffer are allowed.
 * lse       fp32, layout DCP_LSE_BHC (strides l0, l1, l2) or DCP_LSE_BH1
 *           (strides l0, l1; l2 ignored).  lse = -inf marks an empty shard:
 *           its attn rows are never used, whatever they hold (vLLM PR #48897,
 *           port commit: empty shards publish -inf and skip their payload).
 * lse_mode  DCP_LSE_BASE_E or DCP_LSE_BASE_2; the merged LSE is in the same base.
 * out       [B, h_local, D] in the workspace's dtype (fp32 result rounded to
 *           nearest even), row (b, j) at
 *           out + b*out_sb + j*out_sh.  Must not overlap attn.
 * out_lse   [B, h_local] fp32 merged LSE at out_lse + b*out_lse_sb + j, or NULL.
 *
 * A row whose shards are all empty gives out = +0.0 and out_lse = -inf (sglang
 * PR #32851, commit log: such rows give 0, not NaN).  Arithmetic is fp32 in a
 * fixed shard order (ascending; above 16 shards ascending within each group
 * of 16, the groups' sums then added in order) that does not depend on B, the
 * chunking or the launch, so chunked and unchunked calls give identical bits.
 * B = 0 is a no-op.  B > capacity runs ceil(B / capacity) launches over
 * consecutive token ranges, in order, on hip_stream (PR #40539, Modifications).
 *
 * Alignment: attn and out 16-byte aligned; attn_sb, attn_sh, out_sb, out_sh
 * multiples of 8 elements; lse and out_lse 4-byte aligned.  The strides of
 * attn and lse (attn_sb, attn_sh, l0, l1, l2, and h_local times the shard
 * stride) must be below 2^31 elements (DCP_ERR_LAYOUT otherwise): the kernel
 * takes them as 32-bit values.
 */
int dcp_lse_combine(dcp_workspace* ws, const void* attn, int64_t B, int H, int64_t attn_sb, int64_t attn_sh,
                    const float* lse, int lse_layout, int64_t l0, int64_t l1, int64_t l2, int lse_mode, void* out,
                    int64_t out_sb, int64_t out_sh, float* out_lse, int64_t out_lse_sb, void* hip_stream);

/*
 * MLA split-KV decode partials: the producer of the shard partials that
 * dcp_lse_combine merges.  Each DCP shard owns a contiguous slice of the
 * latent KV cache and runs decode attention for every query head over its own
 * tokens, returning the partial output and its LSE ("[DCP] Optimize shared
 * Output, Query, and Indexer/Top-K via peer memory", sglang PR #32851, commit
 * log: KV tokens are owned by DCP ranks and the attention backend returns the
 * LSE for the cross-rank combine).  In the MLA absorbed form the key is the
 * whole 576-column cached row (512 latent + 64 rope columns) and the value is
 * its first 512 columns ("[Attention] Add direct symmetric-memory DCP A2A",
 * vLLM PR #48897, review thread: head_dim = kv_lora_rank = 512).
 *
 * For query row (b, h) and shard s, with the shard's tokens
 * t in [floor(s*T/cp), floor((s+1)*T/cp)):
 *     z_t = softmax_scale * <q[b,h,:], kv[t,:]>          (576 columns)
 *     o_part[b, s*hq + h, :] = sum_t softmax(z)_t * kv[t, 0:512]
 *     lse_part[b, s*hq + h]  = ln sum_t exp(z_t)   (DCP_LSE_BASE_E)
 *                            = log2 sum_t exp(z_t) (DCP_LSE_BASE_2)
 * A shard with no tokens gives o_part = 0 and lse_part = -inf.  The outputs
 * are laid out so that dcp_lse_combine with H = cp*hq, h_local = hq and
 * DCP_LSE_BH1 (l0 = lse_sb, l1 = 1) merges the shards into exact attention
 * over all T tokens.
 *
 * dtype     DCP_DTYPE_BF16 or DCP_DTYPE_FP16: the element type of q, kv and
 *           o_part (the pages' kernels take both).
 * q         [B, hq, 576], row (b, h) at q + b*q_sb + h*q_sh.
 * kv        [T, 576], token t at kv + t*kv_st (one cache shared by all
 *           B query tokens).  May be NULL when T == 0.
 * o_part    [B, cp*hq, 512], row (b, s*hq + h) at o_part + b*o_sb + (s*hq+h)*o_sh.
 * lse_part  [B, cp*hq] fp32 at lse_part + b*lse_sb + s*hq + h.
 * scratch   device buffer of at least dcp_mla_partial_decode_scratch_size()
 *           bytes, 16-byte aligned, for the split-KV partials: when a shard's
 *           keys are split over several workgroups, each split's normalised
 *           output and LSE land here and are merged into o_part / lse_part
 *           by the merge kernel of dcp_lse_combine.  A partial row is stored
 *           in fp16 after multiplication by a power of two that puts its
 *           largest magnitude in [2^14, 2^15), with the inverse factor beside
 *           its LSE, so it keeps 11 significant bits relative to the row's
 *           largest value whatever the values' range (1032 bytes per row).
 *           NULL allowed when the size is 0 (one split per shard).  Contents on
 *           entry are ignored.  A scratch buffer serves one call at a time:
 *           calls that may overlap (on other streams) need buffers of their
 *           own.
 * Arithmetic: MFMA products of the 16-bit inputs with fp32 accumulation for
 * q.k and p.v, fp32 online softmax whose reference maximum is moved only when
 * a score exceeds it by more than 8 (log2 units), so p <= 256; p is rounded
 * to dtype before the p.v product.
 * Alignment: q, kv, o_part 16-byte aligned; q_sb, q_sh, kv_st, o_sb, o_sh
 * multiples of 8 elements; lse_part 4-byte aligned.
 */
int dcp_mla_partial_decode_scratch_size(int64_t B, int hq, int64_t kv_tokens, int cp, size_t* bytes);

int dcp_mla_partial_decode(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                           int64_t kv_tokens, int64_t kv_st, int dtype, int cp, float softmax_scale, int lse_mode,
                           void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part, int64_t lse_sb, void* scratch,
                           size_t scratch_bytes, void* hip_stream);

/*
 * dcp_mla_partial_decode without a scratch argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results (bit for bit), errors
 * and alignment are those of dcp_mla_partial_decode; the split partials go to
 * a static device array of DCP_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends, which fits the
 * partials of every shape this entry point accepts (a shape needing more is
 * rejected with DCP_ERR_WORKSPACE before anything is enqueued).
 *  - The kernels run on hip_stream's device, which must be the current device
 *    (DCP_ERR_STREAM otherwise).  The first call on a device looks up the
 *    array's address there (hipGetSymbolAddress, no allocation), so make that
 *    first call outside graph capture; later calls, captured or not, only
 *    launch kernels.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap on
 *    one GPU (on different streams, or in graphs replayed concurrently) race
 *    and give wrong results.  Calls ordered on one stream are safe; nothing in
 *    the array needs to be cleared between them.
 */
#define DCP_NOALLOC_SCRATCH_BYTES 67368960 /* 510 units x 128 rows x 1032 bytes */

int dcp_mla_partial_decode_noalloc(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                                   int64_t kv_tokens, int64_t kv_st, int dtype, int cp, float softmax_scale,
                                   int lse_mode, void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part,
                                   int64_t lse_sb, void* hip_stream);

/* How dcp_mla_decode_merged reduces the key splits and merges the shards. */
#define DCP_FUSE_NONE 0       /* separate launches: decode, split reduction, shard merge            */
#define DCP_FUSE_EPILOGUE 1   /* one launch: the decode kernel's last arrivals reduce and merge     */
#define DCP_FUSE_AUTO 2       /* the fastest measured on MI355X: REDUCTIONS at >= 16 splits, else NONE */
#define DCP_FUSE_REDUCTIONS 3 /* decode, then one launch that reduces the splits and merges the shards */

/*
 * MLA decode over cp shards followed by the LSE merge of the shards: the
 * per-shard partials of dcp_mla_partial_decode AND their merge, which
 * dcp_lse_combine would compute from them, in one call.  On the pages the
 * merge runs after the partials have made a round trip through global memory
 * and costs a launch per layer; fusing it removes both ("[DCP] Run fi_a2a on
 * FlashInfer's fused all-to-all + LSE reduce", sglang PR #40539, Motivation
 * and commit log).  On one GPU the shards need no exchange, so the merge can
 * run in the decode kernel's epilogue:
 *  - DCP_FUSE_EPILOGUE: every workgroup publishes its part (a split's partial,
 *    or its shard's output) and counts itself in with a device-scope atomic;
 *    the last workgroup of a (row block, shard) to arrive reduces that
 *    shard's key splits, and the last shard of a row block to complete merges
 *    the cp shards into out / out_lse.  No workgroup waits for another.
 *  - DCP_FUSE_NONE: the decode kernel, the split reduction and the shard
 *    merge as separate launches (what dcp_mla_partial_decode followed by
 *    dcp_lse_combine does).
 *  - DCP_FUSE_REDUCTIONS: the decode kernel, then one launch in which each
 *    head's shards are merged, in LDS, by the workgroup that has just
 *    reduced their key splits: no separate shard-merge launch, and o_part is
 *    not read back.  It applies when the shards' keys are split (small B)
 *    and cp <= 16; otherwise it runs as DCP_FUSE_NONE.
 *  - DCP_FUSE_AUTO: the fastest as measured on MI355X (128 heads, 4 shards,
 *    131072 keys, B = 1, 2, 8, 32, 64): REDUCTIONS where the shards' keys
 *    are split 16 ways or more (about 1% faster at B = 1 and 2), else NONE.
 *    The fused epilogue is nowhere faster: at B <= 16 it is slower
 *    (publishing a workgroup's part at agent scope writes back the L2 of its
 *    XCD, and that costs more than the launches it saves), from B = 32 on
 *    even with the separate launches.
 * Every mode gives the same bits: o_part / lse_part equal
 * dcp_mla_partial_decode's, and out / out_lse equal dcp_lse_combine over them
 * (DCP_LSE_BH1, the same lse_mode).
 *
 * q, kv, dtype, cp, softmax_scale, lse_mode, o_part, lse_part: as
 * dcp_mla_partial_decode (o_part / lse_part are outputs here too).
 * out       [B, hq, 512] in dtype, row (b, h) at out + b*out_sb + h*out_sh.
 * out_lse   [B, hq] fp32 at out_lse + b*out_lse_sb + h, or NULL.
 * scratch   device buffer of at least dcp_mla_decode_merged_scratch_size()
 *           bytes, 16-byte aligned, ZERO-FILLED before its first use: it
 *           holds the arrival counters (which every complete call leaves at
 *           zero again, so later calls and graph replays need no clearing)
 *           and the split partials.  One call at a time per buffer.
 * Alignment of out as o_part (16 bytes; strides multiples of 8 elements);
 * out / out_lse must not overlap any other buffer.  Errors as
 * dcp_mla_partial_decode, plus DCP_ERR_INVALID_ARG for an unknown fuse mode.
 */
int dcp_mla_decode_merged_scratch_size(int64_t B, int hq, int64_t kv_tokens, int cp, size_t* bytes);

int dcp_mla_decode_merged(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                          int64_t kv_tokens, int64_t kv_st, int dtype, int cp, float softmax_scale, int lse_mode,
                          void* o_part, int64_t o_sb, int64_t o_sh, float* lse_part, int64_t lse_sb, void* out,
                          int64_t out_sb, int64_t out_sh, float* out_lse, int64_t out_lse_sb, int fuse,
                          void* scratch, size_t scratch_bytes, void* hip_stream);

/*
 * MLA decode partials with one cache per query token and per-token lengths:
 * the producer as a decode batch runs it, each token (request) attending
 * over its own latent KV rows.  The decode seq_lens decide which shards are
 * empty ("[Attention] Add direct symmetric-memory DCP A2A", vLLM PR #48897,
 * amended port commit: the dispatch takes the decode seq_lens and an empty
 * shard publishes LSE = -inf and no payload); with the latent KV spread over
 * the DCP ranks in interleaved order ("[DCP] Optimize shared Output, Query,
 * and Indexer/Top-K via peer memory", sglang PR #32851, commit log) shard s
 * owns every cp-th token of each request.
 *
 * For query row (b, h) let L = min(max(seq_lens[b], 0), max_seq_len) and
 * let R_s be the rows shard s owns (kv_layout: DCP_KV_CONTIGUOUS or
 * DCP_KV_INTERLEAVED, see above); then with z_t = softmax_scale * <q[b,h,:],
 * cache_b[t,:]> over 576 columns,
 *     o_part[b, s*hq + h, :] = sum_{t in R_s} softmax(z)_t * cache_b[t, 0:512]
 *     lse_part[b, s*hq + h]  = log sum_{t in R_s} exp(z_t)  (base of lse_mode)
 * and a shard with R_s empty gives o_part = 0, lse_part = -inf: exactly the
 * input dcp_lse_combine expects, whose merge is attention over all L rows.
 *
 * kv        token b's cache row t at kv + b*kv_sb + t*kv_st (dtype elements);
 *           kv_sb = 0 lets every token share one cache.  Rows t >=
 *           max_seq_len are never read.
 * seq_lens  device int32 [B]; values outside [0, max_seq_len] are clamped.
 * max_seq_len  host bound on seq_lens, used to size the scratch; at most
 *           2^30 (DCP_ERR_INVALID_ARG beyond), so that the device plan
 *           counts keys and tiles exactly in 32 bits.
 * scratch   device buffer of at least
 *           dcp_mla_partial_decode_varlen_scratch_size() bytes (never 0 when
 *           B > 0), 16-byte aligned.  The key splits are sized on the device
 *           from the actual lengths: a planning kernel writes a work list
 *           (longest split first) into the scratch, and splits of a (token,
 *           shard) leave partials there (scaled fp16 rows, as above) that a
 *           reduction kernel merges into o_part / lse_part.  Contents on entry are ignored; one
 *           call at a time per buffer, as for dcp_mla_partial_decode.
 * Other arguments, strides, alignment (kv_sb a multiple of 8 elements too),
 * arithmetic and errors as dcp_mla_partial_decode.  A workgroup serves the
 * heads of one token, so hq below 128 leaves part of each workgroup idle.
 * How the keys are split depends on the lengths of the whole batch, so a
 * token's results can differ in the last bits between batches.
 */
int dcp_mla_partial_decode_varlen_scratch_size(int64_t B, int hq, int64_t max_seq_len, int cp, size_t* bytes);

int dcp_mla_partial_decode_varlen(const void* q, int64_t B, int hq, int64_t q_sb, int64_t q_sh, const void* kv,
                                  int64_t kv_sb, int64_t kv_st, int64_t max_seq_len, const int32_t* seq_lens,
                                  int kv_layout, int dtype, int cp, float softmax_scale, int lse_mode, void* o_part,
                                  int64_t o_sb, int64_t o_sh, float* lse_part, int64_t lse_sb, void* scratch,
                                  size_t scratch_bytes, void* hip_stream);

/*
 * Message for the last failing call on this thread ("" if none): it names the
 * argument at fault and what to change.  The pages report a workspace that
 * cannot be created, or is given a bad configuration, together with the fix
 * ("[DCP] Run fi_a2a on FlashInfer's fused all-to-all + LSE reduce", sglang PR
 * #40539, commit log; "[Attention] Add direct symmetric-memory DCP A2A", vLLM
 * PR #48897, commit messages on the staging-slot count).  The string is owned
 * by the library and stays valid until the next call on the same thread.
 */
const char* dcp_last_error(void);

/* Name of a status code ("DCP_ERR_WORKSPACE", ...; "DCP_ERR_UNKNOWN" for any
 * other value), for the same error reports.  A static string. */
const char* dcp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H */
