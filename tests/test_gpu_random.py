"""Seeded randomized parity sweeps of both entry points against the fp64 oracle.

Each seed draws one configuration from the whole argument space the C ABI
accepts, rather than a shape picked by hand.  For the merge: cp from 1 to 64
(the fixed-cp and the wide kernels), h_local, B (0 included), the workspace
capacity (so 1 to B ordered chunks), both LSE layouts and bases, bf16 or fp16
payloads, padded token and head strides on every tensor, interleaved LSE
strides, empty shards whose payload rows hold NaN, and rows with every shard
empty.  Buffer padding is filled with NaN (inputs) or a sentinel (outputs): a
read of padding poisons the result, a write into it is caught.  For the
producer: the fixed-length and the variable-length entry points with random
B, hq (below, at and above 128 rows per workgroup), cache length (0
included), cp, ownership, lengths (0 and beyond max_seq_len included),
padded strides and either element type.  Tolerances as in test_gpu_merge and
test_gpu_mla.
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


def _strided(shape, strides, dtype, fill):
    """A device view of `shape` with element `strides` inside a buffer filled with `fill`."""
    extent = 1 + sum((n - 1) * s for n, s in zip(shape, strides)) if all(shape) else 1
    buf = torch.full((extent,), fill, dtype=dtype, device=DEV)
    return buf, torch.as_strided(buf, shape, strides)


def _footprint(view):
    """Element offsets (in the backing buffer) that a strided view covers."""
    idx = torch.arange(view.numel(), dtype=torch.int64)
    off = torch.zeros_like(idx)
    rest = idx
    for n, s in reversed(list(zip(view.shape, view.stride()))):
        off += (rest % n) * s
        rest = rest // n
    return off + view.storage_offset()


# ------------------------------------------------------------------------ merge

@pytest.mark.parametrize("seed", range(40))
def test_random_merge(seed):
    rng = np.random.default_rng(10_000 + seed)
    cp = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 32, 48, 64]))
    hl = int(rng.integers(1, max(1, 256 // cp) + 1))
    H = cp * hl
    B = int(rng.integers(0, 49))
    layout = str(rng.choice(["bhc", "bh1"]))
    mode = str(rng.choice(["e", "2"]))
    dtype = torch.float16 if rng.random() < 0.3 else torch.bfloat16
    D = synth.D

    # inputs: payload values, LSEs, empty shards (lse -inf, payload rows NaN)
    g = torch.Generator().manual_seed(seed)
    vals = (torch.randn((B, H, D), generator=g) * float(rng.choice([0.01, 1.0, 30.0]))).to(dtype)
    lo = float(rng.uniform(-40.0, 10.0))
    lse_bhc = torch.from_numpy(rng.uniform(lo, lo + float(rng.uniform(0.0, 40.0)), (B, hl, cp))).float()
    p_empty = float(rng.choice([0.0, 0.1, 0.5]))
    empty = torch.from_numpy(rng.random((B, hl, cp)) < p_empty)
    if B > 2 and rng.random() < 0.5:
        empty[B // 2, hl // 2, :] = True                    # a row with every shard empty
    lse_bhc[empty] = -float("inf")
    for b, j, s in empty.nonzero().tolist():
        vals[b, s * hl + j] = float("nan")                  # never to be used

    sh = D + 8 * int(rng.choice([0, 0, 8, 24]))
    sb = H * sh + 8 * int(rng.choice([0, 0, 16, 40]))
    attn_buf, attn = _strided((B, H, D), (sb, sh, 1), dtype, float("nan"))
    attn.copy_(vals.to(DEV))
    if layout == "bhc":
        l2 = int(rng.choice([1, 2]))
        l1 = cp * l2 + int(rng.choice([0, 3]))
        l0 = hl * l1 + int(rng.choice([0, 5]))
        _, lse = _strided((B, hl, cp), (l0, l1, l2), torch.float32, float("nan"))
        lse.copy_(lse_bhc.to(DEV))
        lse_logical = lse_bhc
    else:
        lse_bh1 = lse_bhc.permute(0, 2, 1).reshape(B, H, 1)  # head s*hl + j
        l1 = int(rng.choice([1, 2]))
        l0 = H * l1 + int(rng.choice([0, 7]))
        _, lse = _strided((B, H, 1), (l0, l1, 1), torch.float32, float("nan"))
        lse.copy_(lse_bh1.to(DEV))
        lse_logical = lse_bh1

    osh = D + 8 * int(rng.choice([0, 8]))
    osb = hl * osh + 8 * int(rng.choice([0, 4]))
    out_buf, out = _strided((B, hl, D), (osb, osh, 1), dtype, 7.0)
    with_lse = rng.random() < 0.8
    olsb = hl + int(rng.choice([0, 3]))
    ol_buf, out_lse = _strided((B, hl), (olsb, 1), torch.float32, 5.0)
    capacity = int(rng.choice([max(B, 1), max(1, B // 3), 1, 1000]))
    wdt = dcp.DCP_DTYPE_FP16 if dtype == torch.float16 else dcp.DCP_DTYPE_BF16
    LAY = {"bhc": dcp.DCP_LSE_BHC, "bh1": dcp.DCP_LSE_BH1}
    MOD = {"e": dcp.DCP_LSE_BASE_E, "2": dcp.DCP_LSE_BASE_2}

    announce("random merge seed=%d B=%d H=%d cp=%d %s/%s %s cap=%d strides attn=(%d,%d) lse=%s out=(%d,%d)" % (
        seed, B, H, cp, layout, mode, synth.payload_name(vals), capacity, sb, sh, tuple(lse.stride()), osb, osh))
    ws = dcp.dcp_workspace_create(capacity, hl, cp, dtype=wdt)
    dcp.dcp_lse_combine(ws, attn, lse, LAY[layout], MOD[mode], out, out_lse if with_lse else None)
    torch.cuda.synchronize()
    ws.close()
    if B == 0:
        assert torch.all(out_buf == 7.0) and torch.all(ol_buf == 5.0)
        return

    case = synth.MergeCase("random seed %d" % seed, vals, lse_logical, cp, layout, mode)
    check_against_oracle(case, out, out_lse if with_lse else None)
    # nothing outside the output views is written
    touched = torch.zeros(out_buf.numel(), dtype=torch.bool)
    touched[_footprint(out)] = True
    assert torch.all(out_buf.cpu()[~touched] == 7.0), "seed %d: the merge wrote outside out" % seed
    lt = torch.zeros(ol_buf.numel(), dtype=torch.bool)
    lt[_footprint(out_lse)] = True
    if with_lse:
        assert torch.all(ol_buf.cpu()[~lt] == 5.0), "seed %d: the merge wrote outside out_lse" % seed
    else:
        assert torch.all(ol_buf.cpu() == 5.0), "seed %d: out_lse written although not passed" % seed

    # one token per launch gives the same bits
    out1 = torch.empty((B, hl, D), dtype=dtype, device=DEV)
    ws1 = dcp.dcp_workspace_create(1, hl, cp, dtype=wdt)
    dcp.dcp_lse_combine(ws1, attn, lse, LAY[layout], MOD[mode], out1, None)
    torch.cuda.synchronize()
    ws1.close()
    assert torch.equal(out1.view(torch.int16), out.contiguous().view(torch.int16))


# --------------------------------------------------------------------- producer

def _check_rows(o_part, lse_part, o_r, l_r, rows, B, hq, cp):
    o_g = o_part.float().cpu().double().numpy().reshape(B, cp, hq, 512)
    l_g = lse_part.cpu().double().numpy().reshape(B, cp, hq)
    for i, r in enumerate(rows):
        b, h = divmod(int(r), hq)
        for s in range(cp):
            og, lg, orr, lr = o_g[b, s, h], l_g[b, s, h], o_r[i, s], l_r[i, s]
            if np.isneginf(lr):
                assert np.isneginf(lg) and np.all(og == 0), "row %d shard %d: empty shard not (0, -inf)" % (r, s)
                continue
            assert abs(lg - lr) <= 1e-5 * max(abs(lr), 1.0), "row %d shard %d: lse %.8g vs %.8g" % (r, s, lg, lr)
            assert np.abs(og - orr).max() <= 2.0 ** -7 * np.abs(orr).max(), "row %d shard %d" % (r, s)


@pytest.mark.parametrize("seed", range(16))
def test_random_producer(seed):
    rng = np.random.default_rng(20_000 + seed)
    varlen = seed % 2 == 1
    B = int(rng.integers(1, 5))
    hq = int(rng.choice([1, 8, 16, 40, 128, 160]))
    cp = int(rng.integers(1, 9))
    T = int(rng.choice([0, 1, 7, 100, 1000, 3000])) if not varlen else int(rng.choice([5, 100, 1000, 3000]))
    dtype = torch.float16 if rng.random() < 0.3 else torch.bfloat16
    mode = dcp.DCP_LSE_BASE_E if rng.random() < 0.5 else dcp.DCP_LSE_BASE_2
    interleaved = bool(rng.random() < 0.5)
    scale = float(rng.choice([synth.MLA_SCALE, 0.02, 0.2]))
    g = torch.Generator().manual_seed(seed)
    q = synth.normal_16((B, hq, 576), g, dtype)
    per_token = varlen and rng.random() < 0.6
    kv = synth.normal_16((B, T, 576) if per_token else (T, 576), g, dtype, std=0.5)

    q_sh = 576 + 8 * int(rng.choice([0, 8]))
    q_sb = hq * q_sh + 8 * int(rng.choice([0, 16]))
    _, q_dev = _strided((B, hq, 576), (q_sb, q_sh, 1), dtype, float("nan"))
    q_dev.copy_(q.to(DEV))
    kv_st = 576 + 8 * int(rng.choice([0, 4]))
    if per_token:
        kv_sb = T * kv_st + 8 * int(rng.choice([0, 32]))
        _, kv_dev = _strided((B, T, 576), (kv_sb, kv_st, 1), dtype, float("nan"))
    else:
        _, kv_dev = _strided((T, 576), (kv_st, 1), dtype, float("nan"))
    if T > 0:
        kv_dev.copy_(kv.to(DEV))
    o_sh = 512 + 8 * int(rng.choice([0, 8]))
    o_sb = cp * hq * o_sh
    _, o_part = _strided((B, cp * hq, 512), (o_sb, o_sh, 1), dtype, float("nan"))
    lse_part = torch.empty((B, cp * hq), dtype=torch.float32, device=DEV)

    if varlen:
        seq = rng.integers(0, T + 1, B).astype(np.int32)
        seq[0] = T
        if B > 1:
            seq[1] = int(rng.choice([0, T + 50, -3]))     # empty, or clamped
        layout = dcp.DCP_KV_INTERLEAVED if interleaved else dcp.DCP_KV_CONTIGUOUS
        nbytes = dcp.dcp_mla_partial_decode_varlen_scratch_size(B, hq, T, cp)
        scratch = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
        announce("random producer (varlen) seed=%d B=%d hq=%d T=%d cp=%d %s layout=%d per_token=%d seq=%s" % (
            seed, B, hq, T, cp, synth.payload_name(q), layout, per_token, list(seq)))
        dcp.dcp_mla_partial_decode_varlen(q_dev, kv_dev, torch.from_numpy(seq).to(DEV), T, layout, cp, scale, mode,
                                          o_part, lse_part, scratch)
    else:
        nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
        scratch = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes else None
        announce("random producer seed=%d B=%d hq=%d T=%d cp=%d %s scratch=%d" % (
            seed, B, hq, T, cp, synth.payload_name(q), nbytes))
        dcp.dcp_mla_partial_decode(q_dev, kv_dev, cp, scale, mode, o_part, lse_part, scratch)
    torch.cuda.synchronize()

    if T == 0:                                            # no keys: every shard is empty
        assert torch.all(torch.isneginf(lse_part)) and torch.all(o_part == 0)
        return
    rows = np.unique(np.concatenate([[0, B * hq - 1], rng.integers(0, B * hq, 14)]))
    if varlen:
        clamped = np.clip(seq.astype(np.int64), 0, T).astype(np.int32)
        o_r, l_r = oracle.attention_partials_varlen(synth.bits16(q), synth.bits16(kv), clamped, cp, scale,
                                                    OMODE[mode], interleaved=interleaved, rows=rows,
                                                    threads=THREADS, dtype=synth.payload_name(q))
    else:
        o_r, l_r = oracle.attention_partials(synth.bits16(q), synth.bits16(kv), cp, scale, OMODE[mode], rows=rows,
                                             threads=THREADS, dtype=synth.payload_name(q))
    _check_rows(o_part, lse_part, o_r, l_r, rows, B, hq, cp)
