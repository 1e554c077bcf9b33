"""GPU parity of dcp_mla_partial_decode (the producer of the shard partials)
against the fp64 oracle, through the C ABI, and of the whole path -- producer
then dcp_lse_combine -- against brute-force full attention.

Tolerances (the pages fix none for the producer; see the oracle's notes):
* per-shard LSE: |L_g - L_r| <= 1e-5 max(|L_r|, 1), -inf exactly;
* per-shard output row: max_d |O_g - O_r| <= 2^-7 max_d |O_r| (p is rounded to
  bf16 before the p.v product, as flash attention does);
* the merge stage: the GPU merge of the GPU's own partials is held to the
  merge tolerance against the oracle merge of those same partials;
* end to end: the merged output within 2^-7 of the row max of fp64 full
  attention over all T keys.
Full-size runs (T = 131072, 128 heads, cp = 4) check every row of the first
and the last token -- each a whole 128-row workgroup, all eight wavefronts and
all sixteen rows of each -- plus sampled rows, which the oracle computes one by
one.
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


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def run_producer(q, kv, cp, scale, mode, q_dev=None, o_part=None):
    B, hq, _ = q.shape
    T = kv.shape[0]
    if q_dev is None:
        q_dev = q.to(DEV)
    kv_dev = kv.to(DEV)
    if o_part is None:
        o_part = torch.empty((B, cp * hq, 512), dtype=q.dtype, device=DEV)
    lse_part = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV) if nbytes else None
    announce("dcp_mla_partial_decode %s B=%d hq=%d T=%d cp=%d mode=%d scratch=%d" % (
        synth.payload_name(q), B, hq, T, cp, mode, nbytes))
    dcp.dcp_mla_partial_decode(q_dev, kv_dev, cp, scale, mode, o_part, lse_part, scratch)
    torch.cuda.synchronize()
    return o_part, lse_part


def check_partials(q, kv, cp, scale, mode, o_part, lse_part, rows=None):
    """Compare the GPU partials of the listed query rows (b*hq + h) with the oracle."""
    B, hq, _ = q.shape
    o_r, l_r = oracle.attention_partials(synth.bits16(q), synth.bits16(kv), cp, scale, OMODE[mode],
                                         rows=rows, threads=THREADS, dtype=synth.payload_name(q))
    rows = np.arange(B * hq) if rows is None else np.asarray(rows)
    o_g = o_part.float().cpu().double().numpy().reshape(B, cp, hq, 512)
    l_g = lse_part.cpu().double().numpy().reshape(B, cp, hq)
    worst = 0.0
    for i, r in enumerate(rows):
        b, h = divmod(int(r), hq)
        for s in range(cp):
            og, lg = o_g[b, s, h], l_g[b, s, h]
            orr, lr = o_r[i, s], l_r[i, s]
            if np.isneginf(lr):
                assert np.isneginf(lg) and np.all(og == 0), "row %d shard %d: empty shard not (0, -inf)" % (r, s)
                continue
            assert abs(lg - lr) <= 1e-5 * max(abs(lr), 1.0), "row %d shard %d: lse %.8g vs %.8g" % (r, s, lg, lr)
            scale_o = np.abs(orr).max()
            err = np.abs(og - orr).max()
            assert err <= 2.0 ** -7 * scale_o, "row %d shard %d: |dO| %.3g > 2^-7 * %.3g" % (r, s, err, scale_o)
            worst = max(worst, err / scale_o)
    return worst


def check_end_to_end(q, kv, cp, scale, mode, o_part, lse_part, rows):
    """Merge the GPU partials with dcp_lse_combine and compare with full attention."""
    B, hq, _ = q.shape
    out = torch.empty((B, hq, 512), dtype=q.dtype, device=DEV)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    ws = dcp.dcp_workspace_create(B, hq, cp,
                                  dtype=dcp.DCP_DTYPE_FP16 if q.dtype == torch.float16 else dcp.DCP_DTYPE_BF16)
    announce("dcp_lse_combine of producer output B=%d hq=%d cp=%d" % (B, hq, cp))
    dcp.dcp_lse_combine(ws, o_part, lse_part, dcp.DCP_LSE_BH1, mode, out, out_lse)
    torch.cuda.synchronize()
    ws.close()
    # merge stage against the oracle merge of the same GPU partials
    case = synth.MergeCase("producer output", o_part.cpu(), lse_part.cpu().reshape(B, cp * hq, 1), cp, "bh1",
                           "e" if mode == dcp.DCP_LSE_BASE_E else "2")
    check_against_oracle(case, out, out_lse)
    # end to end against full attention
    o_f, l_f = oracle.attention_full(synth.bits16(q), synth.bits16(kv), scale, OMODE[mode], rows=rows,
                                     threads=THREADS, dtype=synth.payload_name(q))
    g = out.float().cpu().double().numpy().reshape(B * hq, 512)
    gl = out_lse.cpu().double().numpy().reshape(B * hq)
    for i, r in enumerate(rows):
        assert np.abs(g[r] - o_f[i]).max() <= 2.0 ** -7 * np.abs(o_f[i]).max()
        assert abs(gl[r] - l_f[i]) <= 1e-5 * max(abs(l_f[i]), 1.0)


# ------------------------------------------------------------------ small cases

@pytest.mark.parametrize("mode", [dcp.DCP_LSE_BASE_E, dcp.DCP_LSE_BASE_2])
def test_tiny_two_shards_of_64_rows(mode):
    q, kv = synth.tiny_attention()                     # B=3, 8 heads, T=128, cp=2
    o, l = run_producer(q, kv, 2, synth.MLA_SCALE, mode)
    check_partials(q, kv, 2, synth.MLA_SCALE, mode, o, l)
    check_end_to_end(q, kv, 2, synth.MLA_SCALE, mode, o, l, rows=np.arange(24))


@pytest.mark.parametrize("B,hq,T,cp", [(2, 128, 4096, 4), (1, 128, 16384, 4), (3, 16, 1000, 4), (5, 24, 777, 3)])
def test_split_kv_shapes(B, hq, T, cp):
    """Several splits per shard (scaled fp16 partials + reduction), ragged T, row counts that
    are not a multiple of 64, odd cp."""
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=2000 + T)
    o, l = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([np.arange(min(8, B * hq)), np.arange(B * hq)[-8:],
                                     np.random.default_rng(T).integers(0, B * hq, 16)]))
    check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)
    check_end_to_end(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def _rescaled(q, kv, s):
    """q * 2^-s and kv * 2^s: exact in bf16 (an exponent shift), and every score q.k is unchanged."""
    q2 = (q.float() * 2.0 ** -s).to(q.dtype)
    kv2 = (kv.float() * 2.0 ** s).to(kv.dtype)
    assert torch.equal(q2.float() * 2.0 ** s, q.float()) and torch.equal(kv2.float() * 2.0 ** -s, kv.float())
    return q2, kv2


@pytest.mark.parametrize("s", [20, -20, 60, -60])
def test_split_partials_keep_their_bits_under_power_of_two_rescaling(s):
    """With the cache scaled by 2^s and the queries by 2^-s every score is unchanged and every value is 2^s times
    larger, so o_part must be exactly 2^s times the unscaled result and lse_part identical, bit for bit -- including
    |s| = 60, where the split partials' values (about 2^60 or 2^-60) lie far outside fp16's range: each partial row
    is stored with its own power-of-two factor."""
    B, hq, T, cp = 1, 128, 16384, 4      # 16 splits of 256 keys per shard
    assert dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp) > 0
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=2400)
    o1, l1 = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    q2, kv2 = _rescaled(q, kv, s)
    o2, l2 = run_producer(q2, kv2, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    assert torch.equal(l1, l2)
    assert torch.equal(o2.float() * 2.0 ** -s, o1.float())
    assert torch.isfinite(o2.float()).all()


def test_empty_shards_give_zero_and_minus_inf():
    q, kv = synth.mla_decode(2, T=3, hq=16, seed=77)   # 3 keys over 4 shards: shard 0 is empty
    o, l = run_producer(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2)
    check_partials(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l)
    lh = l.cpu().reshape(2, 4, 16)
    assert torch.all(torch.isneginf(lh[:, 0])) and torch.all(o.cpu().reshape(2, 4, 16, 512)[:, 0] == 0)
    check_end_to_end(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l, rows=np.arange(32))


def test_no_keys_at_all():
    q, kv = synth.mla_decode(2, T=0, hq=16, seed=78)
    o, l = run_producer(q, kv, 2, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    assert torch.all(torch.isneginf(l.cpu())) and torch.all(o.cpu() == 0)


def test_strided_query_and_padded_output():
    B, hq, T, cp = 4, 32, 2048, 4
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=79)
    backing = torch.zeros((B, hq + 16, 576 + 64), dtype=torch.bfloat16)
    backing[:, 8:8 + hq, 32:32 + 576] = q
    qd = backing.to(DEV)[:, 8:8 + hq, 32:32 + 576]
    obuf = torch.full((B, cp * hq + 8, 512 + 64), 5.0, dtype=torch.bfloat16, device=DEV)
    oview = obuf[:, 4:4 + cp * hq, 32:32 + 512]
    o, l = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, q_dev=qd, o_part=oview)
    check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=np.arange(0, B * hq, 5))
    host = obuf.cpu()
    assert torch.all(host[:, :4] == 5.0) and torch.all(host[:, 4 + cp * hq:] == 5.0)
    assert torch.all(host[:, :, :32] == 5.0) and torch.all(host[:, :, 32 + 512:] == 5.0)


def test_largest_kv_row_stride():
    """The cache at the largest row stride the planner accepts ((2^31 - 576) / 32 elements, rounded down to a
    multiple of 8; a 4.4 GB strided view): the tile copies' addresses then reach their largest lane offsets
    (about 2.0e9 bytes) and scalar bases (16 rows apart).  34 keys in one shard: a full first tile and a ragged
    second one, so both copy paths run."""
    B, hq, T, cp = 1, 16, 34, 1
    kv_st = ((((1 << 31) - 576) // 32) // 8) * 8
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=83)
    backing = torch.empty((T - 1) * kv_st + 576, dtype=torch.bfloat16, device=DEV)
    kv_view = backing.as_strided((T, 576), (kv_st, 1))
    kv_view.copy_(kv.to(DEV))
    o_part = torch.empty((B, cp * hq, 512), dtype=q.dtype, device=DEV)
    lse_part = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes else None
    announce("dcp_mla_partial_decode bf16 B=%d hq=%d T=%d cp=%d kv_st=%d (largest accepted)" % (B, hq, T, cp, kv_st))
    dcp.dcp_mla_partial_decode(q.to(DEV), kv_view, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o_part, lse_part, scratch)
    torch.cuda.synchronize()
    del kv_view, backing
    torch.cuda.empty_cache()
    check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o_part, lse_part)


def test_too_small_scratch_is_rejected_before_launch():
    B, hq, T, cp = 1, 128, 8192, 4
    need = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    assert need > 0
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=80)
    o = torch.full((B, cp * hq, 512), 9.0, dtype=torch.bfloat16, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    announce("producer scratch rejection")
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_partial_decode(q.to(DEV), kv.to(DEV), cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, small)
    assert e.value.status == dcp.DCP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o.cpu() == 9.0)


# ------------------------------------------------------------ full-size config

_KV_CACHE = {}


def _full_kv():
    if "kv" not in _KV_CACHE:
        _, kv = synth.mla_decode(1)
        _KV_CACHE["kv"] = kv
    return _KV_CACHE["kv"]


def whole_token_rows(B, hq, seed):
    """Every row of the first and of the last token, plus six random rows."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(hq), np.arange((B - 1) * hq, B * hq), rng.integers(0, B * hq, 6)]))


@pytest.mark.parametrize("B", [1, 8, 32, 64])
def test_full_size_config_whole_tokens(B):
    """q [B,128,576], one 131072 x 576 cache in 4 contiguous shards of 32768,
    scale 1/sqrt(192): all 128 rows of tokens 0 and B-1 (and sampled rows)
    against the oracle, partials and merged."""
    kv = _full_kv()
    q = synth.normal_bf16((B, 128, 576), synth.gen(3000 + B))
    o, l = run_producer(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    rows = whole_token_rows(B, 128, B)
    worst = check_partials(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)
    announce("full size B=%d: %d rows checked, worst partial row error %.3g of row max" % (B, len(rows), worst))
    check_end_to_end(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


# ------------------------------------------------------------- fp16 payloads

F16 = torch.float16


@pytest.mark.parametrize("mode", [dcp.DCP_LSE_BASE_E, dcp.DCP_LSE_BASE_2])
def test_tiny_f16(mode):
    """fp16 q and cache (the pages' other payload type) through the fp16 MFMA."""
    q, kv = synth.tiny_attention(dtype=F16)
    o, l = run_producer(q, kv, 2, synth.MLA_SCALE, mode)
    assert o.dtype == F16
    check_partials(q, kv, 2, synth.MLA_SCALE, mode, o, l)
    check_end_to_end(q, kv, 2, synth.MLA_SCALE, mode, o, l, rows=np.arange(24))


@pytest.mark.parametrize("B,hq,T,cp", [(2, 128, 4096, 4), (5, 24, 777, 3)])
def test_split_kv_shapes_f16(B, hq, T, cp):
    """Several splits per shard: the fp16 per-split partials are reduced by the
    fp16 instance of the merge kernel."""
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=2100 + T, dtype=F16)
    o, l = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    rows = np.unique(np.concatenate([np.arange(min(8, B * hq)), np.arange(B * hq)[-8:],
                                     np.random.default_rng(T).integers(0, B * hq, 16)]))
    check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)
    check_end_to_end(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_empty_shards_f16():
    q, kv = synth.mla_decode(2, T=3, hq=16, seed=177, dtype=F16)
    o, l = run_producer(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2)
    check_partials(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l)
    assert torch.all(torch.isneginf(l.cpu().reshape(2, 4, 16)[:, 0]))


@pytest.mark.parametrize("B", [1, 8, 32, 64])
def test_full_size_config_whole_tokens_f16(B):
    _, kv = synth.mla_decode(1, dtype=F16)
    q = synth.normal_16((B, 128, 576), synth.gen(3100 + B), F16)
    o, l = run_producer(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    rows = whole_token_rows(B, 128, 100 + B)
    worst = check_partials(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)
    announce("full size fp16 B=%d: %d rows checked, worst partial row error %.3g of row max" % (B, len(rows), worst))
    check_end_to_end(q, kv, 4, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=rows)


def test_mixed_element_types_are_rejected():
    q, kv = synth.tiny_attention()
    o = torch.empty((3, 16, 512), dtype=F16, device=DEV)
    l = torch.empty((3, 16), dtype=torch.float32, device=DEV)
    announce("producer with bf16 q and fp16 o_part (rejected in the binding)")
    with pytest.raises(ValueError):
        dcp.dcp_mla_partial_decode(q.to(DEV), kv.to(DEV), 2, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, None)


def test_graph_replays_with_changing_queries_match_eager():
    """The split path (decode kernel + merge over splits) captured in one HIP
    graph and replayed with new query contents, interleaved with eager calls:
    every replay equals the eager call on the same inputs, bit for bit."""
    B, hq, T, cp = 2, 128, 4096, 4
    _, kv = synth.mla_decode(B, T=T, hq=hq, seed=4040)
    kv_dev = kv.to(DEV)
    q_dev = torch.empty((B, hq, 576), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((B, cp * hq, 512), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    assert nbytes > 0
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    q_dev.copy_(synth.normal_bf16((B, hq, 576), synth.gen(4100)).to(DEV))
    torch.cuda.synchronize()
    announce("producer graph capture B=%d hq=%d T=%d cp=%d" % (B, hq, T, cp))
    with torch.cuda.stream(s):
        dcp.dcp_mla_partial_decode(q_dev, kv_dev, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, scratch, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dcp.dcp_mla_partial_decode(q_dev, kv_dev, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, scratch, stream=s)
    torch.cuda.synchronize()
    o_e = torch.empty_like(o)
    l_e = torch.empty_like(l)
    for k in range(3):
        q_dev.copy_(synth.normal_bf16((B, hq, 576), synth.gen(4200 + k)).to(DEV))
        torch.cuda.synchronize()
        announce("producer graph replay %d" % k)
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), l.clone()
        dcp.dcp_mla_partial_decode(q_dev, kv_dev, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o_e, l_e, scratch)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16))
        assert torch.equal(l_g.view(torch.int32), l_e.view(torch.int32))
    q = q_dev.cpu()
    rows = np.arange(0, B * hq, 17)
    check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o_e, l_e, rows=rows)
