"""GPU parity of dcp_mla_partial_decode_varlen against the fp64 oracle.

Each query token attends over its own cache and its own decode length; the
lengths decide which DCP shards are empty ("[Attention] Add direct
symmetric-memory DCP A2A", vLLM PR #48897, amended port commit), and shards
own either a contiguous slice of a token's rows or, with the latent KV spread
over the DCP ranks in interleaved order ("[DCP] Optimize shared Output, Query, and
Indexer/Top-K via peer memory", sglang PR #32851, commit log), every cp-th
row.  Tolerances as for the fixed-length producer (see test_gpu_mla).
"""
import os

import numpy as np
import pytest
import torch

import context_lse_merge_amd as dcp
import oracle
import synth
from tests.merge_helpers import announce, check_against_oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
THREADS = len(os.sched_getaffinity(0))
OMODE = {dcp.DCP_LSE_BASE_E: oracle.BASE_E, dcp.DCP_LSE_BASE_2: oracle.BASE_2}
LAYOUTS = {"contiguous": dcp.DCP_KV_CONTIGUOUS, "interleaved": dcp.DCP_KV_INTERLEAVED}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def run_varlen(q, kv, seq, max_len, layout, cp, mode, kv_dev=None):
    B, hq, _ = q.shape
    o = torch.empty((B, cp * hq, 512), dtype=q.dtype, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    nbytes = dcp.dcp_mla_partial_decode_varlen_scratch_size(B, hq, max_len, cp)
    scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV) if nbytes else None
    announce("dcp_mla_partial_decode_varlen %s B=%d hq=%d max_len=%d layout=%d cp=%d scratch=%d seq=%s" % (
        synth.payload_name(q), B, hq, max_len, layout, cp, nbytes, list(seq[:6])))
    dcp.dcp_mla_partial_decode_varlen(q.to(DEV), kv.to(DEV) if kv_dev is None else kv_dev,
                                      torch.from_numpy(np.asarray(seq, np.int32)).to(DEV), max_len, layout, cp,
                                      synth.MLA_SCALE, mode, o, l, scratch)
    torch.cuda.synchronize()
    return o, l


def check(q, kv, seq, layout, cp, mode, o, l, rows=None):
    B, hq, _ = q.shape
    clamped = np.clip(np.asarray(seq, np.int64), 0, kv.shape[-2]).astype(np.int32)
    o_r, l_r = oracle.attention_partials_varlen(synth.bits16(q), synth.bits16(kv), clamped, cp, synth.MLA_SCALE,
                                                OMODE[mode], interleaved=(layout == dcp.DCP_KV_INTERLEAVED),
                                                rows=rows, threads=THREADS, dtype=synth.payload_name(q))
    rows = np.arange(B * hq) if rows is None else np.asarray(rows)
    o_g = o.float().cpu().double().numpy().reshape(B, cp, hq, 512)
    l_g = l.cpu().double().numpy().reshape(B, cp, hq)
    for i, r in enumerate(rows):
        b, h = divmod(int(r), hq)
        for s in range(cp):
            og, lg, orr, lr = o_g[b, s, h], l_g[b, s, h], o_r[i, s], l_r[i, s]
            if np.isneginf(lr):
                assert np.isneginf(lg) and np.all(og == 0), "row %d shard %d: empty shard not (0, -inf)" % (r, s)
                continue
            assert abs(lg - lr) <= 1e-5 * max(abs(lr), 1.0), "row %d shard %d: lse %.8g vs %.8g" % (r, s, lg, lr)
            assert np.abs(og - orr).max() <= 2.0 ** -7 * np.abs(orr).max(), "row %d shard %d" % (r, s)
    # merged shards (the GPU merge of the GPU partials) against attention over all L rows
    out = torch.empty((B, hq, 512), dtype=q.dtype, device=DEV)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    ws = dcp.dcp_workspace_create(B, hq, cp,
                                  dtype=dcp.DCP_DTYPE_FP16 if q.dtype == torch.float16 else dcp.DCP_DTYPE_BF16)
    dcp.dcp_lse_combine(ws, o, l, dcp.DCP_LSE_BH1, mode, out, out_lse)
    torch.cuda.synchronize()
    ws.close()
    case = synth.MergeCase("varlen output", o.cpu(), l.cpu().reshape(B, cp * hq, 1), cp, "bh1",
                           "e" if mode == dcp.DCP_LSE_BASE_E else "2")
    check_against_oracle(case, out, out_lse)
    o_f, l_f = oracle.attention_partials_varlen(synth.bits16(q), synth.bits16(kv), clamped, 1, synth.MLA_SCALE,
                                                OMODE[mode], rows=rows, threads=THREADS,
                                                dtype=synth.payload_name(q))
    g = out.float().cpu().double().numpy().reshape(B * hq, 512)
    gl = out_lse.cpu().double().numpy().reshape(B * hq)
    for i, r in enumerate(rows):
        if np.isneginf(l_f[i, 0]):
            assert np.all(g[r] == 0) and np.isneginf(gl[r])
            continue
        assert np.abs(g[r] - o_f[i, 0]).max() <= 2.0 ** -7 * np.abs(o_f[i, 0]).max()
        assert abs(gl[r] - l_f[i, 0]) <= 1e-5 * max(abs(l_f[i, 0]), 1.0)


def _caches(seed, B, hq, tmax, dtype=torch.bfloat16):
    g = synth.gen(seed)
    q = synth.normal_16((B, hq, 576), g, dtype)
    kv = synth.normal_16((B, tmax, 576), g, dtype, std=0.5)
    return q, kv


@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
@pytest.mark.parametrize("mode", [dcp.DCP_LSE_BASE_E, dcp.DCP_LSE_BASE_2])
def test_short_and_empty_lengths(layout, mode):
    """Lengths 0, 1, 3 (fewer rows than shards: empty shards), 150 and 300."""
    q, kv = _caches(700, 5, 16, 300)
    seq = [0, 1, 3, 150, 300]
    o, l = run_varlen(q, kv, seq, 300, LAYOUTS[layout], 4, mode)
    check(q, kv, seq, LAYOUTS[layout], 4, mode, o, l)


@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
def test_split_path_long_lengths(layout):
    """Long caches with 128 heads: several key splits per shard, merged by the
    split reduction; lengths that are not multiples of the tile."""
    q, kv = _caches(701, 2, 128, 16384)
    seq = [16384, 9001]
    o, l = run_varlen(q, kv, seq, 16384, LAYOUTS[layout], 4, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(256)[-8:], np.random.default_rng(7).integers(0, 256, 16)]))
    check(q, kv, seq, LAYOUTS[layout], 4, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_heads_not_a_multiple_of_128_and_odd_cp():
    q, kv = _caches(702, 3, 160, 700)
    seq = [700, 2, 333]
    o, l = run_varlen(q, kv, seq, 700, dcp.DCP_KV_INTERLEAVED, 3, dcp.DCP_LSE_BASE_2)
    rows = np.unique(np.concatenate([np.arange(0, 480, 7), [159, 160, 319, 320, 479]]))
    check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, 3, dcp.DCP_LSE_BASE_2, o, l, rows=rows)


def test_lengths_outside_the_range_are_clamped():
    q, kv = _caches(703, 3, 16, 200)
    seq = [-5, 260, 77]                          # read as 0, 200, 77
    o, l = run_varlen(q, kv, seq, 200, dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E)
    check(q, kv, seq, dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E, o, l)
    assert torch.all(torch.isneginf(l.cpu()[0]))


def test_fp16_varlen():
    q, kv = _caches(704, 4, 32, 512, dtype=torch.float16)
    seq = [512, 5, 0, 250]
    o, l = run_varlen(q, kv, seq, 512, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E)
    check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E, o, l)


@pytest.mark.parametrize("B,T", [(2, 4096), (1, 4096), (1, 4000)])
def test_shared_cache_full_length_matches_fixed_length_bitwise(B, T):
    """Every token sharing one cache at its full length, contiguous ownership.
    At these shapes the planning kernel picks the fixed-length path's split
    length (256 keys: 4 splits per shard; T = 4000 ends each shard on a
    partial tile), so every split runs the same tiles in the same order, and
    the split reduction forms the weights exactly as the merge kernel does:
    the same bits.  With B = 1 (a single row block) the fixed-length decode
    runs its two-tiles-in-flight loop and the variable-length one its
    one-tile-ahead loop, so the two loops are checked against each other."""
    q, kv = synth.mla_decode(B, T=T, hq=128, seed=705)
    kv_dev = kv.to(DEV)
    o_v, l_v = run_varlen(q, kv, [T] * B, T, dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E, kv_dev=kv_dev)
    o_f = torch.empty_like(o_v)
    l_f = torch.empty_like(l_v)
    nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, 128, T, 4)
    scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV) if nbytes else None
    announce("fixed-length producer on the same shared cache (B=%d T=%d)" % (B, T))
    dcp.dcp_mla_partial_decode(q.to(DEV), kv_dev, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o_f, l_f, scratch)
    torch.cuda.synchronize()
    assert torch.equal(o_v.view(torch.int16), o_f.view(torch.int16))
    assert torch.equal(l_v.view(torch.int32), l_f.view(torch.int32))


def test_full_size_shared_cache_random_lengths_interleaved():
    """64 tokens over one 131072-row cache (kv_sb = 0) with lengths drawn
    uniformly in [1, 131072], interleaved ownership: every row of two whole
    tokens (the full-length token 0 and the last token) and sampled rows."""
    _, kv = synth.mla_decode(1)
    B = 64
    q = synth.normal_bf16((B, 128, 576), synth.gen(3300))
    seq = np.random.default_rng(3300).integers(1, 131073, B).astype(np.int32)
    seq[:2] = [131072, 3]
    o, l = run_varlen(q, kv, seq, 131072, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(128), [128, 129], np.arange((B - 1) * 128, B * 128),
                                     rng.integers(0, B * 128, 4)]))
    announce("varlen full size: checking %d rows (tokens 0 and %d whole, lengths %d and %d)" % (
        len(rows), B - 1, seq[0], seq[B - 1]))
    check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_split_partials_keep_their_bits_under_power_of_two_rescaling():
    """Per-token caches scaled by 2^s_b (s_b = 40, -40, 0; queries by 2^-s_b): scores are unchanged, so each token's
    o_part rows must be exactly 2^s_b times the unscaled ones and lse_part identical, bit for bit, through the split
    path (scaled fp16 partials in slots, then the split reduction), whatever the values' range."""
    B, hq, T, cp = 3, 128, 12000, 4
    q, kv = _caches(2500, B, hq, T)
    seq = [12000, 9000, 11000]
    assert dcp.dcp_mla_partial_decode_varlen_scratch_size(B, hq, T, cp) > 0
    o1, l1 = run_varlen(q, kv, seq, T, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E)
    sh = [40, -40, 0]
    q2 = torch.stack([(q[b].float() * 2.0 ** -sh[b]).to(q.dtype) for b in range(B)])
    kv2 = torch.stack([(kv[b].float() * 2.0 ** sh[b]).to(kv.dtype) for b in range(B)])
    for b in range(B):
        assert torch.equal(kv2[b].float() * 2.0 ** -sh[b], kv[b].float())
        assert torch.equal(q2[b].float() * 2.0 ** sh[b], q[b].float())
    o2, l2 = run_varlen(q2, kv2, seq, T, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E)
    assert torch.equal(l1, l2)
    for b in range(B):
        assert torch.equal(o2[b].float() * 2.0 ** -sh[b], o1[b].float())


def test_large_batch_of_short_tokens_with_a_few_long_ones():
    """3000 tokens over one 131072-row cache: most lengths in [0, 2000] (some empty), ten full-length tokens whose
    shards are split; 12000 (token, shard) pairs, so every thread of the planning workgroup loops over many pairs and
    the work list holds over 12000 items.  Sampled rows against the oracle, every row through the merge."""
    _, kv = synth.mla_decode(1)
    B, hq, cp = 3000, 16, 4
    q = synth.normal_bf16((B, hq, 576), synth.gen(3400))
    rng = np.random.default_rng(3400)
    seq = rng.integers(0, 2001, B).astype(np.int32)
    long_tokens = rng.choice(B, 10, replace=False)
    seq[long_tokens] = 131072
    seq[:3] = [0, 1, 2000]
    o, l = run_varlen(q, kv, seq, 131072, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([[0, 1, 16, 32, 47, B * hq - 1], long_tokens[:4] * hq + 5,
                                     rng.integers(0, B * hq, 12)]))
    check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_argument_errors():
    q, kv = _caches(706, 2, 16, 64)
    o = torch.empty((2, 64, 512), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((2, 64), dtype=torch.float32, device=DEV)
    seq = torch.tensor([64, 10], dtype=torch.int32, device=DEV)
    announce("varlen argument errors (rejected before launch)")
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_partial_decode_varlen(q.to(DEV), kv.to(DEV), seq, 64, 7, 4, synth.MLA_SCALE,
                                          dcp.DCP_LSE_BASE_E, o, l, None)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        dcp.dcp_mla_partial_decode_varlen(q.to(DEV), kv.to(DEV), seq, 65, dcp.DCP_KV_CONTIGUOUS, 4,
                                          synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, None)


# The split length is chosen on the device from the batch's actual lengths
# (about 256 splits over the whole batch, none under 256 keys), so the cases
# below aim at its regimes: a batch dominated by a few long tokens, a single
# long token split many times per shard, row blocks of a token with more
# than 128 heads, the scratch reused by calls with other lengths, and the
# plan rebuilt on every replay of a captured graph.


def test_skewed_lengths_few_long_tokens():
    """Per-token caches, 3 long tokens among 29 short ones: the long pairs are
    split, the short ones run unsplit, all in one list."""
    B, T = 32, 6144
    q, kv = _caches(707, B, 128, T)
    rng = np.random.default_rng(707)
    seq = rng.integers(0, 300, B).astype(np.int32)
    seq[[3, 17, 30]] = [T, 5000, 4097]
    o, l = run_varlen(q, kv, seq, T, dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([np.arange(3 * 128, 4 * 128, 9), np.arange(17 * 128, 18 * 128, 13),
                                     [30 * 128, 30 * 128 + 127, 0, 1, 5 * 128 + 64, B * 128 - 1]]))
    check(q, kv, seq, dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_one_long_token_many_splits_per_shard():
    """B = 1 over the full 131072-row cache: 4096 tiles, 16-tile splits, so
    64 partials per (shard, head) for the reduction."""
    _, kv = synth.mla_decode(1)
    q = synth.normal_bf16((1, 128, 576), synth.gen(708))
    o, l = run_varlen(q, kv, [131072], 131072, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_2)
    check(q, kv, [131072], dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_2, o, l, rows=[0, 1, 63, 64, 126, 127])


def test_more_than_128_heads_with_splits():
    """hq = 200: two row blocks per token, the second with 72 live rows, and
    pairs split several times."""
    q, kv = _caches(709, 3, 200, 9000)
    seq = [9000, 5, 7001]
    o, l = run_varlen(q, kv, seq, 9000, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([[0, 127, 128, 199, 200, 327, 328, 399, 400, 527, 528, 599],
                                     np.arange(0, 600, 37)]))
    check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_scratch_reused_with_other_lengths_and_repeatable():
    """One scratch buffer, a long-token call, then a call whose plan is
    smaller: the second is right whatever the first left behind, and running
    it again gives the same bits (the list order may differ; the arithmetic
    of each split does not)."""
    B, T = 6, 4096
    q, kv = _caches(710, B, 128, T)
    qd, kvd = q.to(DEV), kv.to(DEV)
    nbytes = dcp.dcp_mla_partial_decode_varlen_scratch_size(B, 128, T, 4)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    outs = []
    for k, seq in enumerate([[4096] * B, [4096, 0, 77, 1000, 2049, 3], [4096, 0, 77, 1000, 2049, 3]]):
        o = torch.empty((B, 4 * 128, 512), dtype=torch.bfloat16, device=DEV)
        l = torch.empty((B, 4 * 128), dtype=torch.float32, device=DEV)
        announce("varlen scratch reuse call %d seq=%s" % (k, seq))
        dcp.dcp_mla_partial_decode_varlen(qd, kvd, torch.tensor(seq, dtype=torch.int32, device=DEV), T,
                                          dcp.DCP_KV_CONTIGUOUS, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l,
                                          scratch)
        torch.cuda.synchronize()
        outs.append((o, l))
    (o1, l1), (o2, l2) = outs[1], outs[2]
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    rows = np.unique(np.concatenate([np.arange(0, B * 128, 23), [128, 255, 5 * 128 + 127]]))
    check(q, kv, [4096, 0, 77, 1000, 2049, 3], dcp.DCP_KV_CONTIGUOUS, 4, dcp.DCP_LSE_BASE_E, o1, l1, rows=rows)


def test_graph_replays_with_changing_lengths_match_eager():
    """The planning kernel, the decode over its list and the split reduction
    captured in one HIP graph; each replay with new seq_lens (and so a new
    plan) equals the eager call on the same inputs, bit for bit."""
    B, T = 4, 4096
    q, kv = _caches(711, B, 128, T)
    qd, kvd = q.to(DEV), kv.to(DEV)
    seq_dev = torch.tensor([4096, 10, 2000, 0], dtype=torch.int32, device=DEV)
    o = torch.empty((B, 4 * 128, 512), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((B, 4 * 128), dtype=torch.float32, device=DEV)
    nbytes = dcp.dcp_mla_partial_decode_varlen_scratch_size(B, 128, T, 4)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def call(o_, l_, stream=None):
        dcp.dcp_mla_partial_decode_varlen(qd, kvd, seq_dev, T, dcp.DCP_KV_INTERLEAVED, 4, synth.MLA_SCALE,
                                          dcp.DCP_LSE_BASE_E, o_, l_, scratch, stream=stream)
    announce("varlen graph capture B=%d T=%d" % (B, T))
    with torch.cuda.stream(s):
        call(o, l, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(o, l, stream=s)
    torch.cuda.synchronize()
    o_e, l_e = torch.empty_like(o), torch.empty_like(l)
    for k, seq in enumerate([[4096, 4096, 4096, 4096], [1, 0, 3000, 4095], [0, 0, 0, 0]]):
        seq_dev.copy_(torch.tensor(seq, dtype=torch.int32))
        torch.cuda.synchronize()
        announce("varlen graph replay %d seq=%s" % (k, seq))
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), l.clone()
        call(o_e, l_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16))
        assert torch.equal(l_g.view(torch.int32), l_e.view(torch.int32))
        if k == 1:
            rows = np.unique(np.concatenate([np.arange(0, B * 128, 29), [B * 128 - 1]]))
            check(q, kv, seq, dcp.DCP_KV_INTERLEAVED, 4, dcp.DCP_LSE_BASE_E, o_e, l_e, rows=rows)
    assert torch.all(torch.isneginf(l_e)) and torch.all(o_e == 0)
