"""GPU parity of dcp_lse_combine against the fp64 oracle, through the C ABI.

Shapes and distributions are the pages' decode geometries (see ``synth``):
the tiny 3-token case, the Kimi-K2.5 geometry (64 heads, cp 4, [B,H/cp,cp]
base-e LSE), the DeepSeek-V2-236B geometry (128 heads, cp 8, FlashMLA
[B,H,1] base-2 LSE), the 512-token stress case with empty shards and 4
ordered chunks, the pages' own test shapes (16 heads x 3 and x 7 tokens with
several calls per batch, 2 heads x 49 tokens; 6 heads per rank at cp 4 out of
a 128-head backing buffer), padded token strides, and every special case the
oracle is pinned on.  Bit-identity is required where the arithmetic is the
same by construction: chunked vs unchunked, either LSE layout, any empty-shard
payload, a common exact LSE shift, cp = 1.
"""
import math

import numpy as np
import pytest
import torch

import synth
from tests.merge_helpers import announce, bf16_ulp, check_against_oracle, gpu_merge, oracle_merge

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _case(name, B, H, cp, layout, mode, seed, lse_lo=-5.0, lse_hi=15.0):
    g = synth.gen(seed)
    attn = synth.normal_bf16((B, H, synth.D), g)
    hl = H // cp
    if layout == "bhc":
        lse = synth.uniform_f32((B, hl, cp), g, lse_lo, lse_hi)
    else:
        lse = synth.uniform_f32((B, H, 1), g, lse_lo, lse_hi)
    return synth.MergeCase(name, attn, lse, cp, layout, mode)


# ----------------------------------------------------------------- the configs

def test_tiny_config():
    c = synth.tiny_merge()
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)


@pytest.mark.parametrize("B", [1, 8, 16, 32, 64, 128, 256, 512])
def test_kimi_geometry(B):
    c = synth.kimi_merge(B)
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_dsv2_geometry_flashmla_lse(B):
    c = synth.dsv2_merge(B)
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)


def test_stress_chunked_with_empty_shards():
    c = synth.stress_merge()
    ref = oracle_merge(c)
    out_c, L_c = gpu_merge(c, capacity=128)            # 4 ordered chunks
    check_against_oracle(c, out_c, L_c, ref=ref)
    out_u, L_u = gpu_merge(c, capacity=512)            # one launch
    assert torch.equal(out_c.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(L_c.view(torch.int32), L_u.view(torch.int32))


# --------------------------------------------------------- pinned special cases

@pytest.mark.parametrize("mode", ["e", "2"])
def test_cp1_is_bit_identity(mode):
    c = _case("cp1", 37, 16, 1, "bhc", mode, 7)
    out, L = gpu_merge(c)
    assert torch.equal(out.cpu().view(torch.int16), c.attn.view(torch.int16))
    assert torch.equal(L.cpu().view(torch.int32), c.lse[:, :, 0].contiguous().view(torch.int32))


@pytest.mark.parametrize("cp", [2, 4, 8])
@pytest.mark.parametrize("mode", ["e", "2"])
def test_equal_lse_gives_mean_within_one_ulp(cp, mode):
    c = _case("equal-lse cp=%d" % cp, 9, 16 * cp, cp, "bhc", mode, 11 + cp)
    c.lse = c.lse[:, :, :1].expand(-1, -1, cp).contiguous()
    out, L = gpu_merge(c)
    B, hl = c.B, c.h_local
    mean = c.attn.double().numpy().reshape(B, cp, hl, synth.D).mean(axis=1)
    g = out.cpu().double().numpy()
    assert np.all(np.abs(g - mean) <= bf16_ulp(mean) + 2.0 ** -16 * np.abs(c.attn.double().numpy()).reshape(
        B, cp, hl, synth.D).mean(axis=1))
    log_cp = math.log(cp) if mode == "e" else math.log2(cp)
    ref = c.lse[:, :, 0].double().numpy() + log_cp
    assert np.all(np.abs(L.cpu().double().numpy() - ref) <= 1e-5 * np.maximum(np.abs(ref), 1))


@pytest.mark.parametrize("mode", ["e", "2"])
def test_common_exact_shift_is_bit_identical(mode):
    c = _case("shift", 33, 64, 4, "bhc", mode, 21, -20, 20)
    c.lse = torch.round(c.lse * 1024) / 1024            # 2^-10 grid: x - M is exact in fp32 before and after
    out0, L0 = gpu_merge(c)
    shifted = synth.MergeCase(c.name + "+64", c.attn, c.lse + 64.0, c.cp, c.lse_layout, c.lse_mode)
    out1, L1 = gpu_merge(shifted)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert np.allclose(L1.cpu().double().numpy(), L0.cpu().double().numpy() + 64.0, rtol=1e-6, atol=0)


def test_base2_and_base_e_agree_after_conversion():
    c = _case("base-e", 20, 64, 4, "bhc", "e", 31, -10, 10)
    c2 = synth.MergeCase("base-2", c.attn, (c.lse.double() * (1 / math.log(2))).float(), 4, "bhc", "2")
    out_e, L_e = gpu_merge(c)
    out_2, L_2 = gpu_merge(c2)
    check_against_oracle(c, out_e, L_e)
    check_against_oracle(c2, out_2, L_2)
    ge, g2 = out_e.cpu().double().numpy(), out_2.cpu().double().numpy()
    assert np.all(np.abs(ge - g2) <= 2 * bf16_ulp(ge) + 2.0 ** -15 * np.abs(ge).max())
    assert np.allclose(L_2.cpu().double().numpy() * math.log(2), L_e.cpu().double().numpy(), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("layout", ["bhc", "bh1"])
def test_one_hot_lse_selects_exact_head(layout):
    """Shard s of local head j is head s*(H/cp) + j: with one non-empty shard the row
    is that head's payload bit for bit."""
    B, H, cp = 11, 64, 4
    hl = H // cp
    g = synth.gen(41)
    attn = synth.normal_bf16((B, H, synth.D), g)
    pick = torch.randint(0, cp, (B, hl), generator=g)
    lse_bhc = torch.full((B, hl, cp), -math.inf)
    lse_bhc.scatter_(2, pick[:, :, None], synth.uniform_f32((B, hl, 1), g, -3, 3))
    lse = lse_bhc if layout == "bhc" else lse_bhc.permute(0, 2, 1).reshape(B, H, 1).contiguous()
    c = synth.MergeCase("one-hot " + layout, attn, lse, cp, layout, "e")
    out, L = gpu_merge(c)
    want = attn[torch.arange(B)[:, None], pick * hl + torch.arange(hl)[None, :]]
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))
    assert torch.equal(L.cpu(), lse_bhc.gather(2, pick[:, :, None])[:, :, 0])


def test_bhc_and_bh1_layouts_are_bit_identical():
    c = synth.dsv2_merge(24)                                   # BH1
    B, H, cp = c.B, c.H, c.cp
    hl = H // cp
    bhc = c.lse.reshape(B, cp, hl).permute(0, 2, 1).contiguous()
    c2 = synth.MergeCase("dsv2 as bhc", c.attn, bhc, cp, "bhc", "2")
    o1, L1 = gpu_merge(c)
    o2, L2 = gpu_merge(c2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32))
    check_against_oracle(c, o1, L1)


def test_empty_shard_payload_is_never_used():
    c = synth.stress_merge(B=96)
    runs = []
    for fill in (float("nan"), float("inf"), -float("inf"), 1e38, 0.0):
        attn = c.attn.clone()
        empty = torch.isnan(attn)
        attn[empty] = fill
        runs.append(gpu_merge(synth.MergeCase(c.name, attn, c.lse, c.cp, "bhc", "e")))
    for o, L in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(L.view(torch.int32), runs[0][1].view(torch.int32))
    check_against_oracle(c, *runs[0])


def test_all_empty_rows_are_zero_and_minus_inf():
    c = _case("all-empty", 6, 32, 4, "bhc", "2", 51)
    c.lse[1] = -math.inf                                   # token 1: every shard empty, all heads
    c.lse[4, 3] = -math.inf                                # token 4, local head 3
    c.attn[1] = float("nan")
    c.attn[4, 3::8] = float("nan")
    out, L = gpu_merge(c)
    assert torch.all(out[1].view(torch.int16) == 0) and torch.all(out[4, 3].view(torch.int16) == 0)
    assert torch.all(torch.isneginf(L[1])) and torch.isneginf(L[4, 3])
    check_against_oracle(c, out, L)


# ------------------------------------------------------------- chunking, shapes

@pytest.mark.parametrize("capacity", [1, 7, 128, 1000])
def test_chunking_is_bit_identical(capacity):
    c = synth.kimi_merge(203)
    o_ref, L_ref = gpu_merge(c, capacity=203)
    o, L = gpu_merge(c, capacity=capacity)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(L.view(torch.int32), L_ref.view(torch.int32))


@pytest.mark.parametrize("cp", [2, 4, 8])
@pytest.mark.parametrize("hl,B,capacity", [(16, 3, 3), (16, 7, 3), (2, 49, 49), (2, 49, 16)])
@pytest.mark.parametrize("mode", ["e", "2"])
def test_pages_test_shapes(cp, hl, B, capacity, mode):
    """16 local heads x 3 tokens, 16 x 7 tokens over several calls, 2 x 49 (the
    pages' reference-equivalence shapes), in both LSE bases."""
    c = _case("pages %dx%d cp=%d cap=%d" % (hl, B, cp, capacity), B, hl * cp, cp, "bhc", mode, 61 + B + cp)
    out, L = gpu_merge(c, capacity=capacity)
    check_against_oracle(c, out, L)
    if capacity < B:
        o1, L1 = gpu_merge(c, capacity=B)
        assert torch.equal(out.view(torch.int16), o1.view(torch.int16))


def test_six_heads_per_rank_in_128_head_backing():
    """6 local heads, cp 4 (H = 24) viewed out of a [B, 128, 512] buffer: a
    non-contiguous token stride of 128 heads."""
    B, cp, hl = 13, 4, 6
    g = synth.gen(71)
    backing = synth.normal_bf16((B, 128, synth.D), g)
    lse = synth.normal_f32((B, 24, 1), g, 3.0, 2.0)
    c = synth.MergeCase("k3 6/rank in 128-head backing", backing[:, :24].contiguous(), lse, cp, "bh1", "e")
    dev_backing = backing.to(DEV)
    view = dev_backing[:, :24]
    assert view.stride(0) == 128 * synth.D
    out, L = gpu_merge(c, attn=view)
    check_against_oracle(c, out, L)
    out2, L2 = gpu_merge(c, attn=view, capacity=4)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_padded_token_and_output_strides_leave_neighbours_untouched():
    B, H, cp = 19, 64, 4
    hl = H // cp
    c = synth.kimi_merge(B)
    padded = torch.full((B, H + 8, synth.D), float("nan"), dtype=torch.bfloat16)
    padded[:, :H] = c.attn
    dev = padded.to(DEV)
    out_buf = torch.full((B, hl + 3, synth.D + 64), 7.0, dtype=torch.bfloat16, device=DEV)
    out_view = out_buf[:, 1:hl + 1, 32:32 + synth.D]
    lse_buf = torch.full((B, hl + 2), 5.0, dtype=torch.float32, device=DEV)
    out, L = gpu_merge(c, attn=dev[:, :H], out=out_view, out_lse=lse_buf[:, 1:hl + 1])
    check_against_oracle(c, out, L)
    host = out_buf.cpu()
    assert torch.all(host[:, 0] == 7.0) and torch.all(host[:, hl + 1:] == 7.0)
    assert torch.all(host[:, :, :32] == 7.0) and torch.all(host[:, :, 32 + synth.D:] == 7.0)
    lh = lse_buf.cpu()
    assert torch.all(lh[:, 0] == 5.0) and torch.all(lh[:, hl + 1:] == 5.0)


@pytest.mark.parametrize("cp", [3, 5, 6, 12, 16, 17, 32, 64])
def test_other_shard_counts(cp):
    hl = 4 if cp > 16 else 8
    c = _case("cp=%d" % cp, 9, hl * cp, cp, "bhc", "e", 81 + cp, -12, 12)
    c.lse[2, 1, cp // 2] = -math.inf
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)
    o2, L2 = gpu_merge(c, capacity=2)
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16))


def test_without_merged_lse():
    c = synth.kimi_merge(10)
    out, _ = gpu_merge(c, with_lse=False)
    check_against_oracle(c, out, None)


def test_element_offsets_beyond_2_31():
    """40000 tokens of 128 heads at cp 8 (a 5.2 GB input): token b starts at
    element b * 65536, past 2^31 from token 32768 on.  The kernel takes the
    strides as 32-bit values and forms every offset in 64 bits; sampled tokens
    on both sides of 2^30 and 2^31, and the last one, against the oracle run
    on just those tokens."""
    import context_lse_merge_amd as dcp
    B, H, cp = 40000, 128, 8
    hl = H // cp
    announce("merge with element offsets past 2^31: B=%d H=%d cp=%d (5.2 GB input)" % (B, H, cp))
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7777)
    attn = torch.empty((B, H, synth.D), dtype=torch.bfloat16, device=DEV)
    for t0 in range(0, B, 4000):
        attn[t0:t0 + 4000] = torch.randn((4000, H, synth.D), generator=gen, device=DEV).to(torch.bfloat16)
    lse = torch.randn((B, H, 1), generator=gen, device=DEV) * 2.0 + 10.0
    out = torch.empty((B, hl, synth.D), dtype=torch.bfloat16, device=DEV)
    out_lse = torch.empty((B, hl), dtype=torch.float32, device=DEV)
    ws = dcp.dcp_workspace_create(B, hl, cp)
    dcp.dcp_lse_combine(ws, attn, lse, dcp.DCP_LSE_BH1, dcp.DCP_LSE_BASE_2, out, out_lse)
    torch.cuda.synchronize()
    ws.close()
    for b in (0, 16383, 16384, 32767, 32768, 32769, B - 1):
        case = synth.MergeCase("token %d of %d" % (b, B), attn[b:b + 1].cpu(), lse[b:b + 1].cpu(), cp, "bh1", "2")
        check_against_oracle(case, out[b:b + 1], out_lse[b:b + 1])
    del attn


def test_zero_tokens_is_a_no_op():
    import context_lse_merge_amd as dcp
    ws = dcp.dcp_workspace_create(4, 16, 4)
    attn = torch.empty((0, 64, synth.D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, 16, synth.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((0, 16, 4), dtype=torch.float32, device=DEV)
    dcp.dcp_lse_combine(ws, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out)
    torch.cuda.synchronize()
    ws.close()


def test_one_workspace_reused_across_batch_sizes():
    """One workspace (capacity 64) serves calls of B = 64, 3, 130 (3 ordered
    chunks), 1 and 64 again, in that order on its stream; each call matches the
    oracle and the repeated B = 64 call gives the same bits as the first."""
    import context_lse_merge_amd as dcp
    ws = dcp.dcp_workspace_create(64, 16, 4)
    try:
        first = None
        for k, B in enumerate([64, 3, 130, 1, 64]):
            c = synth.kimi_merge(B)
            attn, lse = c.attn.to(DEV), c.lse.to(DEV)
            out = torch.empty((B, 16, synth.D), dtype=torch.bfloat16, device=DEV)
            L = torch.empty((B, 16), dtype=torch.float32, device=DEV)
            announce("workspace reuse call %d: B=%d capacity=64" % (k, B))
            dcp.dcp_lse_combine(ws, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out, L)
            torch.cuda.synchronize()
            check_against_oracle(c, out, L)
            if B == 64:
                if first is None:
                    first = (out.clone(), L.clone())
                else:
                    assert torch.equal(out.view(torch.int16), first[0].view(torch.int16))
                    assert torch.equal(L.view(torch.int32), first[1].view(torch.int32))
    finally:
        ws.close()


@pytest.mark.parametrize("which", ["kimi", "dsv2", "stress", "kimi_f16"])
def test_cached_load_policy_gives_identical_bits(which):
    """DCP_LOAD_CACHED (plain loads and stores) against the default streaming
    policy on the same inputs: identical bits, including NaN-filled empty shards."""
    import context_lse_merge_amd as dcp
    c = {"kimi": lambda: synth.kimi_merge(96), "dsv2": lambda: synth.dsv2_merge(40),
         "stress": lambda: synth.stress_merge(300), "kimi_f16": lambda: synth.kimi_merge(96, dtype=torch.float16)}[which]()
    dtype = dcp.DCP_DTYPE_FP16 if c.attn.dtype == torch.float16 else dcp.DCP_DTYPE_BF16
    attn, lse = c.attn.to(DEV), c.lse.to(DEV)
    layout = dcp.DCP_LSE_BHC if c.lse_layout == "bhc" else dcp.DCP_LSE_BH1
    mode = dcp.DCP_LSE_BASE_E if c.lse_mode == "e" else dcp.DCP_LSE_BASE_2
    results = []
    for policy in (dcp.DCP_LOAD_STREAMING, dcp.DCP_LOAD_CACHED):
        ws = dcp.dcp_workspace_create(c.capacity or c.B, c.h_local, c.cp, dtype=dtype)
        dcp.dcp_workspace_set_load_policy(ws, policy)
        out = torch.empty((c.B, c.h_local, synth.D), dtype=c.attn.dtype, device=DEV)
        L = torch.empty((c.B, c.h_local), dtype=torch.float32, device=DEV)
        announce("load policy %d on %s" % (policy, c.name))
        dcp.dcp_lse_combine(ws, attn, lse, layout, mode, out, L)
        torch.cuda.synchronize()
        ws.close()
        results.append((out, L))
    check_against_oracle(c, results[1][0], results[1][1])
    assert torch.equal(results[0][0].view(torch.int16), results[1][0].view(torch.int16))
    assert torch.equal(results[0][1].view(torch.int32), results[1][1].view(torch.int32))


# ------------------------------------------------------------ streams and graphs

def test_call_on_another_stream_is_rejected_before_launch():
    import context_lse_merge_amd as dcp
    c = synth.kimi_merge(4)
    attn, lse = c.attn.to(DEV), c.lse.to(DEV)
    out = torch.full((4, 16, synth.D), 3.0, dtype=torch.bfloat16, device=DEV)
    ws = dcp.dcp_workspace_create(8, 16, 4)                 # bound to the current (default) stream
    other = torch.cuda.Stream()
    announce("stream rejection")
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_lse_combine(ws, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out, stream=other)
    assert e.value.status == dcp.DCP_ERR_STREAM
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 3.0)                      # nothing ran
    ws.close()


def test_argument_errors_with_real_buffers():
    import context_lse_merge_amd as dcp
    c = synth.kimi_merge(4)
    attn, lse = c.attn.to(DEV), c.lse.to(DEV)
    out = torch.zeros((4, 16, synth.D), dtype=torch.bfloat16, device=DEV)
    ws = dcp.dcp_workspace_create(8, 16, 4)
    announce("argument errors")
    with pytest.raises(dcp.DcpError) as e:                  # out aliases the input
        dcp.dcp_lse_combine(ws, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, attn[:, :16])
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG
    with pytest.raises(dcp.DcpError) as e:                  # 8-byte offset breaks the 16-byte rule
        flat = torch.zeros(4 * 64 * synth.D + 4, dtype=torch.bfloat16, device=DEV)
        mis = flat[4:].view(4, 64, synth.D)
        dcp.dcp_lse_combine(ws, mis, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out)
    assert e.value.status == dcp.DCP_ERR_ALIGN
    ws12 = dcp.dcp_workspace_create(8, 12, 4)
    with pytest.raises(dcp.DcpError) as e:                  # H / cp = 16 but the workspace holds 12 local heads
        dcp.dcp_lse_combine(ws12, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out)
    assert e.value.status == dcp.DCP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 0)
    ws.close()
    ws12.close()


def test_graph_replays_with_changing_inputs_interleaved_with_eager():
    import context_lse_merge_amd as dcp
    B = 40
    cases = [synth.kimi_merge(B, seed=500 + k) for k in range(4)]
    attn = cases[0].attn.to(DEV)
    lse = cases[0].lse.to(DEV)
    out = torch.empty((B, 16, synth.D), dtype=torch.bfloat16, device=DEV)
    out_lse = torch.empty((B, 16), dtype=torch.float32, device=DEV)
    cap_stream = torch.cuda.Stream()
    ws_graph = dcp.dcp_workspace_create(16, 16, 4, stream=cap_stream)   # 3 chunks inside the graph
    ws_eager = dcp.dcp_workspace_create(B, 16, 4)
    graph = torch.cuda.CUDAGraph()
    announce("graph capture of dcp_lse_combine (3 chunks)")
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap_stream):
        dcp.dcp_lse_combine(ws_graph, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out, out_lse,
                            stream=cap_stream)
    for k, c in enumerate(cases):
        attn.copy_(c.attn.to(DEV))
        lse.copy_(c.lse.to(DEV))
        announce("graph replay %d" % k)
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_lse = out.clone(), out_lse.clone()
        e_out, e_lse = gpu_merge(c)                                       # eager, another workspace and stream
        assert torch.equal(g_out.view(torch.int16), e_out.view(torch.int16))
        assert torch.equal(g_lse.view(torch.int32), e_lse.view(torch.int32))
        check_against_oracle(c, g_out, g_lse)
        # an eager call through the eager workspace between replays
        dcp.dcp_lse_combine(ws_eager, attn, lse, dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, torch.empty_like(out))
        torch.cuda.synchronize()
    ws_graph.close()
    ws_eager.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_staged_merge_in_the_workspace_landing_zone(dtype):
    """A caller gathers the shards into the workspace's landing zone -- each shard's [B, h_local, D] head slice and
    its LSEs copied in from a buffer of its own, as an exchange would deliver them -- and merges them there.  A batch
    wider than the capacity is staged and merged chunk by chunk.  The result meets the oracle and equals the in-place
    merge of the same values bit for bit."""
    import context_lse_merge_amd as dcp
    B, cap = 150, 64
    c = synth.kimi_merge(B, dtype=dtype)
    hl, cp = c.h_local, c.cp
    ref_out, ref_lse = gpu_merge(c)                      # in place, one launch
    shards = [c.attn[:, s * hl:(s + 1) * hl].contiguous().to(DEV) for s in range(cp)]
    shard_lse = [c.lse[:, :, s].contiguous().to(DEV) for s in range(cp)]     # BHC [B, hl, cp] -> per shard [B, hl]
    wdt = dcp.DCP_DTYPE_FP16 if dtype == torch.float16 else dcp.DCP_DTYPE_BF16
    ws = dcp.dcp_workspace_create(cap, hl, cp, dtype=wdt)
    assert ws.buf.numel() == dcp.dcp_workspace_size(cap, hl, cp, dtype=wdt)
    r_attn, r_lse = dcp.dcp_workspace_recv(ws)
    assert tuple(r_attn.shape) == (cap, cp * hl, synth.D) and tuple(r_lse.shape) == (cap, cp * hl)
    out = torch.empty((B, hl, synth.D), dtype=dtype, device=DEV)
    out_lse = torch.empty((B, hl), dtype=torch.float32, device=DEV)
    announce("staged merge through the landing zone: %s B=%d capacity=%d" % (synth.payload_name(c.attn), B, cap))
    for t0 in range(0, B, cap):
        n = min(cap, B - t0)
        r_attn[:n].fill_(float("nan"))                   # stale contents are overwritten by the staging below
        for s in range(cp):
            r_attn[:n, s * hl:(s + 1) * hl].copy_(shards[s][t0:t0 + n])
            r_lse[:n, s * hl:(s + 1) * hl].copy_(shard_lse[s][t0:t0 + n])
        dcp.dcp_lse_combine(ws, r_attn[:n], r_lse[:n], dcp.DCP_LSE_BH1, dcp.DCP_LSE_BASE_E, out[t0:t0 + n],
                            out_lse[t0:t0 + n])
    torch.cuda.synchronize()
    ws.close()
    check_against_oracle(c, out, out_lse)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(out_lse.view(torch.int32), ref_lse.view(torch.int32))
