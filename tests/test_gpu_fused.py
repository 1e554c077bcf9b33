"""dcp_mla_decode_merged: the producer with the split reduction and the shard
merge fused into its epilogue (DCP_FUSE_EPILOGUE), or run as separate launches
(DCP_FUSE_NONE), or with the two reductions in one launch after the decode
(DCP_FUSE_REDUCTIONS), or chosen by shape (DCP_FUSE_AUTO).

Every mode must give the same bits as the unfused pipeline --
dcp_mla_partial_decode followed by dcp_lse_combine over its partials (FlashMLA
layout) -- since all of them run the merge's one row arithmetic; and the merged
output must meet the oracle (the merge tolerance against the oracle merge of
the GPU's own partials, and 2^-7 of the row maximum against fp64 attention over
all keys).  The arrival counters live in the scratch buffer, which is zeroed
once and left zero by every call: repeated calls, calls in other modes and graph
replays on one scratch buffer must keep giving the unfused pipeline's bits.
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
MODES = {"none": dcp.DCP_FUSE_NONE, "epilogue": dcp.DCP_FUSE_EPILOGUE, "reductions": dcp.DCP_FUSE_REDUCTIONS,
         "auto": dcp.DCP_FUSE_AUTO}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _dt(q):
    return dcp.DCP_DTYPE_FP16 if q.dtype == torch.float16 else dcp.DCP_DTYPE_BF16


def unfused(qd, kvd, cp, mode):
    """dcp_mla_partial_decode, then dcp_lse_combine over its partials."""
    B, hq, _ = qd.shape
    T = kvd.shape[0]
    o = torch.empty((B, cp * hq, 512), dtype=qd.dtype, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    n = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    scratch = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    dcp.dcp_mla_partial_decode(qd, kvd, cp, synth.MLA_SCALE, mode, o, l, scratch)
    out = torch.empty((B, hq, 512), dtype=qd.dtype, device=DEV)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    ws = dcp.dcp_workspace_create(max(B, 1), hq, cp, dtype=_dt(qd))
    dcp.dcp_lse_combine(ws, o, l, dcp.DCP_LSE_BH1, mode, out, out_lse)
    torch.cuda.synchronize()
    ws.close()
    return o, l, out, out_lse


def merged(qd, kvd, cp, mode, fuse, scratch=None, stream=None):
    B, hq, _ = qd.shape
    o = torch.full((B, cp * hq, 512), 3.0, dtype=qd.dtype, device=DEV)
    l = torch.full((B, cp * hq), 3.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, hq, 512), 3.0, dtype=qd.dtype, device=DEV)
    out_lse = torch.full((B, hq), 3.0, dtype=torch.float32, device=DEV)
    dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, mode, o, l, out, out_lse, fuse=fuse, scratch=scratch,
                              stream=stream)
    torch.cuda.synchronize()
    return o, l, out, out_lse


def same_bits(x, y):
    if x.dtype == torch.float32:
        return torch.equal(x.view(torch.int32), y.view(torch.int32))
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


def assert_all_equal(got, ref, what):
    for name, g, r in zip(("o_part", "lse_part", "out", "out_lse"), got, ref):
        assert same_bits(g, r), "%s: %s differs from the unfused pipeline" % (what, name)


# (B, hq, T, cp): 16 splits per shard (fixed-cp split reduction), 64 splits (the wide one), 8, one split, a partial
# row block, 2 splits with odd cp, row blocks that span tokens (hq = 160, 6 splits), empty shards, no keys.
SHAPES = [(2, 128, 16384, 4), (1, 128, 65536, 4), (8, 128, 32768, 4), (64, 128, 2048, 4), (3, 16, 1000, 4),
          (5, 24, 777, 3), (3, 160, 3000, 2), (2, 16, 3, 4), (2, 16, 0, 2)]


@pytest.mark.parametrize("B,hq,T,cp", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_every_mode_equals_the_unfused_pipeline(B, hq, T, cp, dtype):
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=9100 + T, dtype=dtype)
    qd, kvd = q.to(DEV), kv.to(DEV)
    mode = dcp.DCP_LSE_BASE_E if (B + T) % 2 else dcp.DCP_LSE_BASE_2
    nsplit_scratch = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    announce("merged producer %s B=%d hq=%d T=%d cp=%d mode=%d (split scratch %d)" % (
        synth.payload_name(q), B, hq, T, cp, mode, nsplit_scratch))
    ref = unfused(qd, kvd, cp, mode)
    scratch = torch.zeros(dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp) or 16, dtype=torch.uint8, device=DEV)
    for name, fuse in MODES.items():
        announce("  fuse=%s" % name)
        got = merged(qd, kvd, cp, mode, fuse, scratch=scratch)
        assert_all_equal(got, ref, "fuse=%s" % name)
    cnt = dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp) - nsplit_scratch
    assert cnt >= 0 and torch.all(scratch[:cnt] == 0), "the arrival counters were not left at zero"


def test_repeated_calls_and_graph_replays_on_one_scratch():
    """Eight splits per shard: calls with new queries, alternating modes, then a captured fused call replayed with
    new queries between eager calls -- every result equals the unfused pipeline on the same inputs."""
    B, hq, T, cp = 8, 128, 32768, 4
    q0, kv = synth.mla_decode(B, T=T, hq=hq, seed=9200)
    kvd = kv.to(DEV)
    qd = torch.empty_like(q0, device=DEV)
    scratch = torch.zeros(dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp), dtype=torch.uint8, device=DEV)
    for k, fuse in enumerate([dcp.DCP_FUSE_EPILOGUE, dcp.DCP_FUSE_REDUCTIONS, dcp.DCP_FUSE_NONE,
                              dcp.DCP_FUSE_EPILOGUE, dcp.DCP_FUSE_REDUCTIONS]):
        qd.copy_(synth.normal_bf16((B, hq, 576), synth.gen(9300 + k)).to(DEV))
        announce("merged producer repeated call %d fuse=%d" % (k, fuse))
        assert_all_equal(merged(qd, kvd, cp, dcp.DCP_LSE_BASE_E, fuse, scratch=scratch),
                         unfused(qd, kvd, cp, dcp.DCP_LSE_BASE_E), "call %d" % k)
    s = torch.cuda.Stream()
    o = torch.empty((B, cp * hq, 512), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    out = torch.empty((B, hq, 512), dtype=torch.bfloat16, device=DEV)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)

    for fuse in (dcp.DCP_FUSE_EPILOGUE, dcp.DCP_FUSE_REDUCTIONS):
        def call():
            dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, out, out_lse,
                                      fuse=fuse, scratch=scratch, stream=s)

        with torch.cuda.stream(s):
            call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        announce("merged producer graph capture, fuse=%d" % fuse)
        with torch.cuda.graph(g, stream=s):
            call()
        torch.cuda.synchronize()
        for k in range(3):
            qd.copy_(synth.normal_bf16((B, hq, 576), synth.gen(9400 + k)).to(DEV))
            torch.cuda.synchronize()
            announce("merged producer graph replay %d" % k)
            g.replay()
            torch.cuda.synchronize()
            assert_all_equal((o.clone(), l.clone(), out.clone(), out_lse.clone()),
                             unfused(qd, kvd, cp, dcp.DCP_LSE_BASE_E), "replay %d" % k)
            assert_all_equal(merged(qd, kvd, cp, dcp.DCP_LSE_BASE_E, fuse, scratch=scratch),
                             unfused(qd, kvd, cp, dcp.DCP_LSE_BASE_E), "eager after replay %d" % k)
        del g
    assert torch.all(scratch[:dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp)
                             - dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)] == 0)


@pytest.mark.parametrize("cp", [4, 16])
def test_combined_reductions_without_out_lse(cp):
    """DCP_FUSE_REDUCTIONS with out_lse = NULL, at 4 shards and at the largest shard count it takes (16: one block
    of 16 wavefronts per head): o_part, lse_part and out equal the unfused pipeline's bits."""
    B, hq, T = 3, 40, 8192
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=9700 + cp)
    qd, kvd = q.to(DEV), kv.to(DEV)
    assert dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp) > 0, "the shape must split the shards' keys"
    announce("merged producer, combined reductions, cp=%d, out_lse NULL" % cp)
    ref = unfused(qd, kvd, cp, dcp.DCP_LSE_BASE_2)
    o = torch.full((B, cp * hq, 512), 3.0, dtype=qd.dtype, device=DEV)
    l = torch.full((B, cp * hq), 3.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, hq, 512), 3.0, dtype=qd.dtype, device=DEV)
    scratch = torch.zeros(dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp), dtype=torch.uint8, device=DEV)
    dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l, out, None,
                              fuse=dcp.DCP_FUSE_REDUCTIONS, scratch=scratch)
    torch.cuda.synchronize()
    for name, g, r in zip(("o_part", "lse_part", "out"), (o, l, out), ref[:3]):
        assert same_bits(g, r), "%s differs from the unfused pipeline" % name


@pytest.mark.parametrize("B,T", [(2, 16384), (32, 32768)])
def test_fused_output_against_the_oracle(B, T):
    """The fused path's merged output: the merge tolerance against the oracle merge of the GPU's own partials (all
    rows), and 2^-7 of the row maximum against fp64 attention over all keys (whole first and last tokens)."""
    hq, cp = 128, 4
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=9500 + B)
    announce("merged producer vs oracle B=%d T=%d" % (B, T))
    o, l, out, out_lse = merged(q.to(DEV), kv.to(DEV), cp, dcp.DCP_LSE_BASE_E, dcp.DCP_FUSE_EPILOGUE)
    case = synth.MergeCase("fused merged output", o.cpu(), l.cpu().reshape(B, cp * hq, 1), cp, "bh1", "e")
    check_against_oracle(case, out, out_lse)
    rows = np.concatenate([np.arange(hq), np.arange((B - 1) * hq, B * hq)]) if B > 1 else np.arange(hq)
    o_f, l_f = oracle.attention_full(synth.bits16(q), synth.bits16(kv), synth.MLA_SCALE, oracle.BASE_E, rows=rows,
                                     threads=THREADS)
    g = out.float().cpu().double().numpy().reshape(B * hq, 512)
    gl = out_lse.cpu().double().numpy().reshape(B * hq)
    worst = 0.0
    for i, r in enumerate(rows):
        err = np.abs(g[r] - o_f[i]).max() / np.abs(o_f[i]).max()
        assert err <= 2.0 ** -7, "row %d: %.3g of the row maximum" % (r, err)
        assert abs(gl[r] - l_f[i]) <= 1e-5 * max(abs(l_f[i]), 1.0)
        worst = max(worst, err)
    announce("merged producer vs fp64 attention: %d rows, worst %.3g of the row maximum" % (len(rows), worst))


def test_errors_are_reported_before_anything_runs():
    B, hq, T, cp = 2, 128, 16384, 4
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=9600)
    qd, kvd = q.to(DEV), kv.to(DEV)
    need = dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp)
    o = torch.full((B, cp * hq, 512), 9.0, dtype=torch.bfloat16, device=DEV)
    l = torch.full((B, cp * hq), 9.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, hq, 512), 9.0, dtype=torch.bfloat16, device=DEV)
    small = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    announce("merged producer error paths")
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, out, None,
                                  fuse=dcp.DCP_FUSE_EPILOGUE, scratch=small)
    assert e.value.status == dcp.DCP_ERR_WORKSPACE and "dcp_mla_decode_merged_scratch_size" in str(e.value)
    scratch = torch.zeros(need, dtype=torch.uint8, device=DEV)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, out, None, fuse=7,
                                  scratch=scratch)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG
    with pytest.raises(dcp.DcpError) as e:       # out inside o_part
        dcp.dcp_mla_decode_merged(qd, kvd, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, o[:, :hq], None,
                                  scratch=scratch)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(o.cpu() == 9.0) and torch.all(out.cpu() == 9.0) and torch.all(scratch.cpu() == 0)
