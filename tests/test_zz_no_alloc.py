"""dcp_mla_partial_decode_noalloc (split partials in the library's static
device array) against dcp_mla_partial_decode with a caller-provided scratch
buffer: the same kernels on the same inputs, so the outputs must agree bit for
bit.  Calls run back to back, each later one on a smaller input than the one
before, so that what an earlier call left in the shared array cannot leak into
a later result.
"""
import pytest
import torch

import context_lse_merge_amd as dcp
import synth
from tests.merge_helpers import announce

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _with_scratch(q, kv, cp, mode):
    B, hq, _ = q.shape
    T = kv.shape[0]
    o = torch.empty((B, cp * hq, 512), dtype=q.dtype, device=DEV)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)
    n = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    scratch = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    dcp.dcp_mla_partial_decode(q, kv, cp, synth.MLA_SCALE, mode, o, l, scratch)
    return o, l, n


def _noalloc(q, kv, cp, mode):
    B, hq, _ = q.shape
    o = torch.full((B, cp * hq, 512), 7.0, dtype=q.dtype, device=DEV)
    l = torch.full((B, cp * hq), 7.0, dtype=torch.float32, device=DEV)
    dcp.dcp_mla_partial_decode_noalloc(q, kv, cp, synth.MLA_SCALE, mode, o, l)
    return o, l


# (B, hq, T, cp): the first needs exactly DCP_NOALLOC_SCRATCH_BYTES (255 row-block x shard units,
# two splits each), each later one less than the one before; the last has a single split (no scratch).
SEQUENCE = [(51, 128, 2560, 5), (2, 128, 16384, 4), (1, 64, 4096, 4), (3, 16, 1000, 3), (64, 128, 2048, 4)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_noalloc_matches_scratch_entry_point_over_shrinking_calls(dtype):
    needs = []
    for k, (B, hq, T, cp) in enumerate(SEQUENCE):
        q, kv = synth.mla_decode(B, T=T, hq=hq, seed=7100 + k, dtype=dtype)
        qd, kvd = q.to(DEV), kv.to(DEV)
        mode = dcp.DCP_LSE_BASE_E if k % 2 == 0 else dcp.DCP_LSE_BASE_2
        announce("noalloc call %d: %s B=%d hq=%d T=%d cp=%d" % (k, synth.payload_name(q), B, hq, T, cp))
        o_ref, l_ref, n = _with_scratch(qd, kvd, cp, mode)
        o_na, l_na = _noalloc(qd, kvd, cp, mode)
        torch.cuda.synchronize()
        needs.append(n)
        assert n <= dcp.DCP_NOALLOC_SCRATCH_BYTES
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), "call %d: o_part differs" % k
        assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32)), "call %d: lse_part differs" % k
    assert needs[0] == dcp.DCP_NOALLOC_SCRATCH_BYTES
    assert all(a > b for a, b in zip(needs, needs[1:])) and needs[-1] == 0


def test_noalloc_repeated_call_on_a_smaller_input_matches():
    """Two calls in a row, the second on a smaller input, each against the scratch entry point."""
    for k, (B, T) in enumerate([(4, 8192), (1, 3000)]):
        q, kv = synth.mla_decode(B, T=T, hq=128, seed=7200 + k)
        qd, kvd = q.to(DEV), kv.to(DEV)
        announce("noalloc repeat %d: B=%d T=%d" % (k, B, T))
        o_na, l_na = _noalloc(qd, kvd, 4, dcp.DCP_LSE_BASE_E)
        o_ref, l_ref, n = _with_scratch(qd, kvd, 4, dcp.DCP_LSE_BASE_E)
        torch.cuda.synchronize()
        assert n > 0
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32))
