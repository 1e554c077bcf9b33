"""GPU parity of dcp_lse_combine with fp16 payloads against the fp64 oracle.

The pages' merge kernels take fp16 as well as bf16 partials (sglang PR
#40539, Motivation: fp16/bf16 only; vLLM PR #48897, port commit: both output
dtypes).  The same configurations as the bf16 suite, with the attention
output drawn in fp32 and rounded to IEEE binary16, through a workspace
created with DCP_DTYPE_FP16; the tolerance is the bf16 one with the fp16 ulp
(2 ulp_f16(r) + 2^-16 A, ulp_f16(r) = 2^(max(floor(log2|r|), -14) - 10)).
Plus what only fp16 has: subnormal payloads and values near its 65504
maximum.
"""
import math

import numpy as np
import pytest
import torch

import context_lse_merge_amd as dcp
import synth
from tests.merge_helpers import announce, check_against_oracle, f16_ulp, gpu_merge

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
F16 = torch.float16


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def test_tiny_config_f16():
    c = synth.tiny_merge(dtype=F16)
    out, L = gpu_merge(c)
    assert out.dtype == F16
    check_against_oracle(c, out, L)


@pytest.mark.parametrize("B", [1, 8, 64, 128, 512])
def test_kimi_geometry_f16(B):
    c = synth.kimi_merge(B, dtype=F16)
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)


@pytest.mark.parametrize("B", [1, 16, 64, 512])
def test_dsv2_geometry_flashmla_lse_f16(B):
    c = synth.dsv2_merge(B, dtype=F16)
    out, L = gpu_merge(c)
    check_against_oracle(c, out, L)


def test_stress_chunked_with_empty_shards_f16():
    """10% empty (token, shard) pairs whose payload is NaN (0x7E00 in fp16), LSE
    spread U[-30, 30], 4 ordered chunks; identical bits to one unchunked launch."""
    c = synth.stress_merge(dtype=F16)
    assert torch.isnan(c.attn).any()
    out, L = gpu_merge(c, capacity=c.capacity)
    check_against_oracle(c, out, L)
    out1, L1 = gpu_merge(c, capacity=c.B)
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(L.view(torch.int32), L1.view(torch.int32))


@pytest.mark.parametrize("capacity", [1, 7, 128])
def test_chunking_is_bit_identical_f16(capacity):
    c = synth.kimi_merge(203, dtype=F16)
    o_ref, L_ref = gpu_merge(c, capacity=203)
    o, L = gpu_merge(c, capacity=capacity)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(L.view(torch.int32), L_ref.view(torch.int32))


def test_cp1_is_bit_identity_f16():
    g = synth.gen(71)
    attn = synth.normal_16((19, 16, synth.D), g, F16)
    lse = synth.uniform_f32((19, 16, 1), g, -5, 15)
    c = synth.MergeCase("cp1 fp16", attn, lse, 1, "bhc", "e")
    out, L = gpu_merge(c)
    assert torch.equal(out.cpu().view(torch.int16), attn.view(torch.int16))
    assert torch.equal(L.cpu().view(torch.int32), lse[:, :, 0].contiguous().view(torch.int32))


@pytest.mark.parametrize("cp", [2, 8])
def test_equal_lse_gives_mean_f16(cp):
    g = synth.gen(80 + cp)
    B, hl = 9, 16
    attn = synth.normal_16((B, hl * cp, synth.D), g, F16)
    lse = synth.uniform_f32((B, hl, 1), g, -5, 15).expand(-1, -1, cp).contiguous()
    c = synth.MergeCase("equal-lse fp16 cp=%d" % cp, attn, lse, cp, "bhc", "2")
    out, L = gpu_merge(c)
    O = attn.double().numpy().reshape(B, cp, hl, synth.D)
    mean = O.mean(axis=1)
    got = out.cpu().double().numpy()
    assert np.all(np.abs(got - mean) <= f16_ulp(mean) + 2.0 ** -16 * np.abs(O).mean(axis=1))
    ref = lse[:, :, 0].double().numpy() + math.log2(cp)
    assert np.all(np.abs(L.cpu().double().numpy() - ref) <= 1e-5 * np.maximum(np.abs(ref), 1))


def test_subnormal_and_near_max_payloads_f16():
    """Payloads of magnitude 2^-20 (fp16 subnormals) in some rows and up to 6e4 in
    others: widening is exact, the fp32 merge neither underflows the subnormals
    nor overflows near the fp16 maximum, and narrowing rounds to nearest even."""
    g = synth.gen(91)
    B, H, cp = 6, 32, 4
    base = torch.randn((B, H, synth.D), generator=g, dtype=torch.float32)
    scale = torch.tensor([2.0 ** -20, 2.0 ** -16, 1.0, 1.0e3, 3.0e4, 6.0e4])[:, None, None]
    attn = (base.clamp(-1.0, 1.0) * scale).to(F16)
    lse = synth.uniform_f32((B, H // cp, cp), g, -3.0, 3.0)
    c = synth.MergeCase("fp16 subnormal and near-max", attn, lse, cp, "bhc", "e")
    assert (attn[0].abs() < 2.0 ** -14).all() and attn[5].abs().max() > 3.0e4
    out, L = gpu_merge(c)
    assert torch.isfinite(out.float()).all()
    check_against_oracle(c, out, L)


def test_payload_dtype_must_match_the_workspace():
    c = synth.kimi_merge(4)                          # bf16 payload
    ws = dcp.dcp_workspace_create(4, 16, 4, dtype=dcp.DCP_DTYPE_FP16)
    try:
        out = torch.empty((4, 16, synth.D), dtype=torch.bfloat16, device=DEV)
        announce("fp16 workspace given bf16 tensors (rejected in the binding)")
        with pytest.raises(ValueError):
            dcp.dcp_lse_combine(ws, c.attn.to(DEV), c.lse.to(DEV), dcp.DCP_LSE_BHC, dcp.DCP_LSE_BASE_E, out)
    finally:
        ws.close()
