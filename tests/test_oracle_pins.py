"""Pins for the fp64 oracle, each against something other than the oracle itself.

The oracle (``oracle/oracle.c``) must be right before anything is compared to
it.  These CPU tests tie it to what the pages and the mathematics fix:

* hand-derived closed forms (``tests/golden/merge_closed_forms.txt``);
* special cases: cp = 1 is the identity, equal LSEs give the mean, a common
  LSE shift changes nothing, base 2 and base e agree after conversion
  (the pages' two LSE bases, sglang PR #40539 Modifications / Accuracy Tests);
* the head mapping h = s*(H/cp) + j (PR #40539 Modifications) by one-hot LSEs,
  and the equivalence of the [B,H/cp,cp] and FlashMLA [B,H,1] layouts;
* empty shards: LSE = -inf and a payload that is never read (vLLM PR #48897
  port commit), an all-empty row giving 0 (sglang PR #32851 commit log);
* library routines (scipy's softmax and logsumexp, numpy matmul) for the
  general merge and for brute-force softmax attention;
* the split-softmax identity itself: merging per-shard attention partials
  reproduces full attention over the concatenated KV; associativity and
  shard-permutation symmetry of the merge.

A dropped term, a wrong sign, a transposed index or a wrong base anywhere in
the oracle fails at least one of these (``test_oracle_mutants`` checks that
claim by planting such mistakes in a copy of ``oracle.c``).
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "merge_closed_forms.txt")
LN2 = math.log(2.0)


def _parse_golden(path):
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0], "o": []}
            elif key == "mode":
                cur["mode"] = oracle.BASE_E if vals[0] == "e" else oracle.BASE_2
            elif key == "lse":
                cur["lse"] = [float(v) for v in vals]
            elif key == "o":
                cur["o"].append([float(v) for v in vals])
            elif key == "out":
                cur["out"] = [float(v) for v in vals]
            elif key == "L":
                cur["L"] = float(vals[0])
            elif key == "end":
                cases.append(cur)
                cur = None
    return cases


GOLDEN_CASES = _parse_golden(GOLDEN)


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c["name"] for c in GOLDEN_CASES])
def test_golden_closed_forms(case):
    cp = len(case["lse"])
    O = np.array(case["o"], dtype=np.float64)[None]           # [1, cp (= H, H_local = 1), D]
    lse = np.array(case["lse"], dtype=np.float64).reshape(1, 1, cp)
    out, L, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, case["mode"])
    np.testing.assert_allclose(out[0, 0], case["out"], rtol=1e-13, atol=1e-300)
    assert not np.isnan(out).any()
    if math.isinf(case["L"]):
        assert L[0, 0] == case["L"]
    else:
        assert abs(L[0, 0] - case["L"]) <= 1e-13 * max(1.0, abs(case["L"]))


def test_all_empty_output_is_positive_zero():
    O = np.full((1, 2, 3), np.nan)
    lse = np.full((1, 1, 2), -np.inf)
    out, L, _ = oracle.merge(O, lse, 2, oracle.LSE_BHC, oracle.BASE_2)
    assert np.all(out == 0.0) and not np.signbit(out).any()
    assert L[0, 0] == -np.inf


def test_bf16_decode_matches_torch():
    special = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x0000, 0x7F7F, 0x3E00], np.uint16)
    got = oracle.bf16_to_f64(special)
    ref = torch.from_numpy(special.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref)
    assert got[0] == 1.0 and got[1] == -2.0 and got[4] == 2.0 ** -133
    bits = np.random.default_rng(7).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_decode_matches_numpy_for_every_bit_pattern():
    """The oracle's own IEEE binary16 decode against numpy's float16 -> float64
    conversion, exhaustively: all 65536 patterns (zeros, subnormals, normals,
    infinities, NaNs)."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan]) and np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x3C00] == 1.0 and got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0


def test_f16_entry_equals_f64_entry():
    rng = np.random.default_rng(11)
    O16 = rng.standard_normal((3, 16, 64)).astype(np.float16)
    lse = rng.uniform(-5, 15, size=(3, 8, 2)).astype(np.float32)
    out_h, L_h, A_h = oracle.merge(O16.view(np.uint16), lse, 2, oracle.LSE_BHC, oracle.BASE_E, dtype="f16")
    out_d, L_d, A_d = oracle.merge(O16.astype(np.float64), lse.astype(np.float64), 2, oracle.LSE_BHC, oracle.BASE_E)
    assert np.array_equal(out_h, out_d) and np.array_equal(L_h, L_d) and np.array_equal(A_h, A_d)


def _random_case(rng, B, H, cp, D=512):
    O = rng.standard_normal((B, H, D))
    lse = rng.uniform(-5, 15, size=(B, H // cp, cp))
    return O, lse


def test_bf16_entry_equals_f64_entry():
    c = synth.tiny_merge()
    bits = synth.bf16_bits(c.attn)
    out_b, L_b, A_b = oracle.merge(bits, c.lse.numpy(), c.cp, oracle.LSE_BHC, oracle.BASE_E)
    O64 = c.attn.double().numpy()
    out_d, L_d, A_d = oracle.merge(O64, c.lse.double().numpy(), c.cp, oracle.LSE_BHC, oracle.BASE_E)
    assert np.array_equal(out_b, out_d) and np.array_equal(L_b, L_d) and np.array_equal(A_b, A_d)


@pytest.mark.parametrize("mode", [oracle.BASE_E, oracle.BASE_2])
def test_cp1_is_identity(mode):
    c = synth.kimi_merge(5)
    bits = synth.bf16_bits(c.attn)
    lse = c.lse.reshape(5, 64, 1)[:, :, :1].contiguous().numpy()  # [B, H, 1], cp = 1
    out, L, _ = oracle.merge(bits, lse, 1, oracle.LSE_BHC, mode)
    assert np.array_equal(out, c.attn.double().numpy())
    assert np.array_equal(L, lse[:, :, 0].astype(np.float64))


@pytest.mark.parametrize("cp", [2, 4, 8])
@pytest.mark.parametrize("mode", [oracle.BASE_E, oracle.BASE_2])
def test_equal_lse_gives_mean(cp, mode):
    rng = np.random.default_rng(cp)
    B, hl, D = 3, 5, 64
    O = rng.standard_normal((B, hl * cp, D))
    lse = np.repeat(rng.uniform(-4, 4, size=(B, hl, 1)), cp, axis=2)
    out, L, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, mode)
    mean = O.reshape(B, cp, hl, D).mean(axis=1)          # shard s holds heads s*hl .. s*hl+hl-1
    np.testing.assert_allclose(out, mean, rtol=1e-14, atol=1e-15)
    log_cp = math.log(cp) if mode == oracle.BASE_E else math.log2(cp)
    np.testing.assert_allclose(L, lse[:, :, 0] + log_cp, rtol=1e-15)


@pytest.mark.parametrize("mode", [oracle.BASE_E, oracle.BASE_2])
def test_common_shift_is_invariant(mode):
    rng = np.random.default_rng(11)
    B, hl, cp, D = 4, 6, 4, 32
    O = rng.standard_normal((B, hl * cp, D))
    lse = np.round(rng.uniform(-20, 20, size=(B, hl, cp)) * 1024) / 1024    # 2^-10 grid: shifts are exact
    out0, L0, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, mode)
    out1, L1, _ = oracle.merge(O, lse + 64.0, cp, oracle.LSE_BHC, mode)
    assert np.array_equal(out0, out1)
    np.testing.assert_allclose(L1, L0 + 64.0, rtol=1e-15)


def test_base2_equals_base_e_after_conversion():
    rng = np.random.default_rng(12)
    O, lse_e = _random_case(rng, 3, 32, 4, D=64)
    out_e, L_e, _ = oracle.merge(O, lse_e, 4, oracle.LSE_BHC, oracle.BASE_E)
    out_2, L_2, _ = oracle.merge(O, lse_e / LN2, 4, oracle.LSE_BHC, oracle.BASE_2)
    np.testing.assert_allclose(out_2, out_e, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L_2 * LN2, L_e, rtol=1e-13)


@pytest.mark.parametrize("cp,mode", [(2, oracle.BASE_E), (4, oracle.BASE_2), (8, oracle.BASE_E), (3, oracle.BASE_2)])
def test_general_merge_matches_scipy_softmax(cp, mode):
    rng = np.random.default_rng(100 + cp)
    B, hl, D = 4, 3, 40
    O = rng.standard_normal((B, hl * cp, D))
    lse = rng.uniform(-30, 30, size=(B, hl, cp))
    out, L, A = oracle.merge(O, lse, cp, oracle.LSE_BHC, mode)
    nat = lse if mode == oracle.BASE_E else lse * LN2       # base-2 LSE in natural-log units
    p = softmax(nat, axis=2)                                 # [B, hl, cp]
    Os = O.reshape(B, cp, hl, D).transpose(0, 2, 1, 3)      # [B, hl, cp, D], shard axis from heads
    ref = np.einsum("bjs,bjsd->bjd", p, Os)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A, np.einsum("bjs,bjsd->bjd", p, np.abs(Os)), rtol=1e-12, atol=1e-13)
    refL = logsumexp(nat, axis=2)
    if mode == oracle.BASE_2:
        refL = refL / LN2
    np.testing.assert_allclose(L, refL, rtol=1e-13)


@pytest.mark.parametrize("layout", [oracle.LSE_BHC, oracle.LSE_BH1])
def test_one_hot_lse_selects_head_group(layout):
    """Shard s of local head j is head s*(H/cp) + j: with only shard s* non-empty the
    output row is exactly that head's payload."""
    rng = np.random.default_rng(3)
    B, H, cp, D = 5, 24, 4, 16
    hl = H // cp
    O = rng.standard_normal((B, H, D))
    pick = rng.integers(0, cp, size=(B, hl))
    lse_bhc = np.full((B, hl, cp), -np.inf)
    for b in range(B):
        for j in range(hl):
            lse_bhc[b, j, pick[b, j]] = rng.uniform(-3, 3)
    lse = lse_bhc if layout == oracle.LSE_BHC else lse_bhc.transpose(0, 2, 1).reshape(B, H)
    out, L, _ = oracle.merge(O, lse, cp, layout, oracle.BASE_E)
    for b in range(B):
        for j in range(hl):
            assert np.array_equal(out[b, j], O[b, pick[b, j] * hl + j])
            assert L[b, j] == lse_bhc[b, j, pick[b, j]]


def test_bhc_and_bh1_layouts_agree():
    c = synth.dsv2_merge(4)
    bits = synth.bf16_bits(c.attn)
    B, H, cp = c.B, c.H, c.cp
    hl = H // cp
    lse_bh1 = c.lse.numpy().reshape(B, H)
    lse_bhc = lse_bh1.reshape(B, cp, hl).transpose(0, 2, 1).copy()     # (b, j, s) = head s*hl + j
    a = oracle.merge(bits, lse_bh1, cp, oracle.LSE_BH1, oracle.BASE_2)
    b = oracle.merge(bits, lse_bhc, cp, oracle.LSE_BHC, oracle.BASE_2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_empty_shards_equal_merge_without_them():
    rng = np.random.default_rng(21)
    B, hl, cp, D = 6, 4, 4, 32
    O = rng.standard_normal((B, hl * cp, D))
    lse = rng.uniform(-10, 10, size=(B, hl, cp))
    empty = rng.random((B, cp)) < 0.35
    empty[0] = [True, True, True, False]
    empty[1] = [True, True, True, True]        # an all-empty token
    for b in range(B):
        for s in range(cp):
            if empty[b, s]:
                lse[b, :, s] = -np.inf
                O[b, s * hl:(s + 1) * hl] = np.nan
    out, L, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, oracle.BASE_E)
    assert not np.isnan(out).any()
    for b in range(B):
        keep = [s for s in range(cp) if not empty[b, s]]
        for j in range(hl):
            if not keep:
                assert np.all(out[b, j] == 0.0) and L[b, j] == -np.inf
                continue
            p = softmax(lse[b, j, keep])
            ref = sum(p[i] * O[b, s * hl + j] for i, s in enumerate(keep))
            np.testing.assert_allclose(out[b, j], ref, rtol=1e-12, atol=1e-13)
            assert abs(L[b, j] - logsumexp(lse[b, j, keep])) <= 1e-13 * max(1, abs(L[b, j]))


def test_stress_case_has_no_nan_and_matches_scipy():
    c = synth.stress_merge(B=64)
    bits = synth.bf16_bits(c.attn)
    out, L, _ = oracle.merge(bits, c.lse.numpy(), c.cp, oracle.LSE_BHC, oracle.BASE_E)
    assert not np.isnan(out).any()
    lse = c.lse.double().numpy()
    O = c.attn.double().numpy()
    hl = c.h_local
    for b in range(0, 64, 7):
        for j in range(0, hl, 5):
            keep = [s for s in range(c.cp) if lse[b, j, s] != -np.inf]
            if not keep:
                continue
            p = softmax(lse[b, j, keep])
            ref = sum(p[i] * O[b, s * hl + j] for i, s in enumerate(keep))
            np.testing.assert_allclose(out[b, j], ref, rtol=1e-12, atol=1e-13)


def test_merge_is_associative():
    rng = np.random.default_rng(31)
    B, hl, D = 3, 5, 24
    O = rng.standard_normal((B, 3 * hl, D))
    lse = rng.uniform(-8, 8, size=(B, hl, 3))
    out3, L3, _ = oracle.merge(O, lse, 3, oracle.LSE_BHC, oracle.BASE_E)
    out_ab, L_ab, _ = oracle.merge(O[:, :2 * hl], lse[:, :, :2].copy(), 2, oracle.LSE_BHC, oracle.BASE_E)
    O2 = np.concatenate([out_ab, O[:, 2 * hl:]], axis=1)
    lse2 = np.stack([L_ab, lse[:, :, 2]], axis=2)
    out_2, L_2, _ = oracle.merge(O2, lse2, 2, oracle.LSE_BHC, oracle.BASE_E)
    np.testing.assert_allclose(out_2, out3, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L_2, L3, rtol=1e-13)


def test_merge_is_symmetric_in_shards():
    rng = np.random.default_rng(41)
    B, hl, cp, D = 3, 4, 8, 16
    O = rng.standard_normal((B, hl * cp, D))
    lse = rng.uniform(-8, 8, size=(B, hl, cp))
    perm = rng.permutation(cp)
    Op = O.reshape(B, cp, hl, D)[:, perm].reshape(B, cp * hl, D)
    out, L, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, oracle.BASE_2)
    outp, Lp, _ = oracle.merge(Op, lse[:, :, perm].copy(), cp, oracle.LSE_BHC, oracle.BASE_2)
    np.testing.assert_allclose(outp, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lp, L, rtol=1e-14)


# ---------------------------------------------------------------- attention

def _scipy_attention(q_bits, kv_bits, scale, t0, t1, dv=512):
    """Decode attention by library routines: numpy matmul for the scores,
    scipy softmax/logsumexp for the normalisation."""
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    kv = torch.from_numpy(kv_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    B, hq, dqk = q.shape
    k = kv[t0:t1]
    z = scale * (q.reshape(B * hq, dqk) @ k.T)                # [rows, t]
    if t1 <= t0:
        return np.zeros((B * hq, dv)), np.full(B * hq, -np.inf)
    return softmax(z, axis=1) @ k[:, :dv], logsumexp(z, axis=1)


def test_f16_attention_matches_scipy():
    """fp16 q and KV (the pages' other payload type): the oracle's per-shard
    partials and full attention against numpy/scipy on the fp16 values."""
    g = synth.gen(515)
    q = synth.normal_16((2, 4, synth.D_QK), g, torch.float16)
    kv = synth.normal_16((96, synth.D_QK), g, torch.float16, std=0.5)
    qb, kb = synth.bits16(q), synth.bits16(kv)
    qd = qb.view(np.float16).astype(np.float64).reshape(8, synth.D_QK)
    kd = kb.view(np.float16).astype(np.float64)
    z = synth.MLA_SCALE * (qd @ kd.T)
    o, lse = oracle.attention_full(qb, kb, synth.MLA_SCALE, oracle.BASE_E, dtype="f16")
    np.testing.assert_allclose(o, softmax(z, axis=1) @ kd[:, :512], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-13)
    op, lp = oracle.attention_partials(qb, kb, 3, synth.MLA_SCALE, oracle.BASE_2, dtype="f16")
    for s, (t0, t1) in enumerate([(0, 32), (32, 64), (64, 96)]):
        zz = z[:, t0:t1]
        np.testing.assert_allclose(op[:, s], softmax(zz, axis=1) @ kd[t0:t1, :512], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lp[:, s], logsumexp(zz, axis=1) / LN2, rtol=1e-13)


def _varlen_case(seed, B, hq, tmax, dtype=torch.bfloat16):
    g = synth.gen(seed)
    q = synth.normal_16((B, hq, synth.D_QK), g, dtype)
    kv = synth.normal_16((B, tmax, synth.D_QK), g, dtype, std=0.5)
    return q, kv


def _owned_rows(L, cp, s, interleaved):
    if interleaved:
        return np.arange(s, L, cp)
    return np.arange((s * L) // cp, ((s + 1) * L) // cp)


@pytest.mark.parametrize("interleaved", [False, True])
def test_varlen_partials_match_scipy(interleaved):
    """One cache per token, seq_lens 0, 1, 3 (< cp), 37 and 100 (= Tmax): each
    shard's partial against numpy/scipy over exactly the rows it owns; shards
    that own nothing are -inf and 0."""
    B, hq, tmax, cp = 5, 2, 100, 4
    q, kv = _varlen_case(601, B, hq, tmax)
    seq = np.array([0, 1, 3, 37, 100], np.int32)
    o, lse = oracle.attention_partials_varlen(synth.bf16_bits(q), synth.bf16_bits(kv), seq, cp, synth.MLA_SCALE,
                                              oracle.BASE_E, interleaved=interleaved)
    qd, kd = q.double().numpy(), kv.double().numpy()
    for b in range(B):
        for h in range(hq):
            r = b * hq + h
            for s in range(cp):
                own = _owned_rows(int(seq[b]), cp, s, interleaved)
                if own.size == 0:
                    assert np.isneginf(lse[r, s]) and np.all(o[r, s] == 0)
                    continue
                z = synth.MLA_SCALE * (kd[b, own] @ qd[b, h])
                np.testing.assert_allclose(o[r, s], softmax(z) @ kd[b, own, :512], rtol=1e-11, atol=1e-13)
                assert abs(lse[r, s] - logsumexp(z)) <= 1e-12 * max(1.0, abs(logsumexp(z)))


@pytest.mark.parametrize("interleaved", [False, True])
def test_varlen_merged_shards_equal_full_attention(interleaved):
    """Merging the shards of a token (oracle merge, BH1 layout) gives attention
    over all its seq_lens[b] rows, whichever way the rows are owned."""
    B, hq, tmax, cp = 4, 3, 64, 8
    q, kv = _varlen_case(602, B, hq, tmax)
    seq = np.array([64, 5, 1, 29], np.int32)
    o, lse = oracle.attention_partials_varlen(synth.bf16_bits(q), synth.bf16_bits(kv), seq, cp, synth.MLA_SCALE,
                                              oracle.BASE_2, interleaved=interleaved)
    O = o.reshape(B, hq, cp, 512).transpose(0, 2, 1, 3).reshape(B, cp * hq, 512)   # head s*hq + h
    L = lse.reshape(B, hq, cp).transpose(0, 2, 1).reshape(B, cp * hq)
    out, Lm, _ = oracle.merge(O, L, cp, oracle.LSE_BH1, oracle.BASE_2)
    qd, kd = q.double().numpy(), kv.double().numpy()
    for b in range(B):
        n = int(seq[b])
        z = synth.MLA_SCALE * (qd[b] @ kd[b, :n].T)                 # [hq, n]
        np.testing.assert_allclose(out[b], softmax(z, axis=1) @ kd[b, :n, :512], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(Lm[b], logsumexp(z, axis=1) / LN2, rtol=1e-12)


def test_varlen_with_one_shared_cache_equals_contiguous_partials():
    """All tokens sharing one cache with seq_lens = T and contiguous ownership is
    exactly the fixed-length producer's computation."""
    q, kv = synth.tiny_attention(B=3, hq=4, T=130)
    seq = np.full(3, 130, np.int32)
    o_v, l_v = oracle.attention_partials_varlen(synth.bf16_bits(q), synth.bf16_bits(kv), seq, 4, synth.MLA_SCALE,
                                                oracle.BASE_E)
    o_f, l_f = oracle.attention_partials(synth.bf16_bits(q), synth.bf16_bits(kv), 4, synth.MLA_SCALE, oracle.BASE_E)
    assert np.array_equal(o_v, o_f) and np.array_equal(l_v, l_f)


def test_full_attention_matches_scipy():
    q, kv = synth.tiny_attention(B=2, hq=4, T=96)
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(kv)
    o, lse = oracle.attention_full(qb, kb, synth.MLA_SCALE, oracle.BASE_E)
    ro, rl = _scipy_attention(qb, kb, synth.MLA_SCALE, 0, 96)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13)
    o2, lse2 = oracle.attention_full(qb, kb, synth.MLA_SCALE, oracle.BASE_2)
    np.testing.assert_allclose(o2, o, rtol=0, atol=0)
    np.testing.assert_allclose(lse2 * LN2, rl, rtol=1e-13)


@pytest.mark.parametrize("T,cp", [(128, 2), (256, 4), (130, 4), (3, 4)])
def test_partials_are_softmax_over_contiguous_shards(T, cp):
    q, kv = synth.tiny_attention(B=2, hq=3, T=T)
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(kv)
    o, lse = oracle.attention_partials(qb, kb, cp, synth.MLA_SCALE, oracle.BASE_E)
    for s in range(cp):
        t0, t1 = (s * T) // cp, ((s + 1) * T) // cp
        ro, rl = _scipy_attention(qb, kb, synth.MLA_SCALE, t0, t1)
        np.testing.assert_allclose(o[:, s], ro, rtol=1e-11, atol=1e-13)
        if t1 > t0:
            np.testing.assert_allclose(lse[:, s], rl, rtol=1e-13)
        else:
            assert np.all(lse[:, s] == -np.inf) and np.all(o[:, s] == 0.0)


@pytest.mark.parametrize("T,cp,mode", [(128, 2, oracle.BASE_E), (256, 4, oracle.BASE_2), (130, 4, oracle.BASE_E),
                                       (3, 4, oracle.BASE_2)])
def test_merged_partials_equal_full_attention(T, cp, mode):
    """The split-softmax identity the DCP merge rests on: merging per-shard
    softmax partials by their LSE gives softmax attention over all KV rows."""
    q, kv = synth.tiny_attention(B=3, hq=8, T=T)
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(kv)
    o_p, l_p = oracle.attention_partials(qb, kb, cp, synth.MLA_SCALE, mode)
    n = o_p.shape[0]
    O = o_p.transpose(1, 0, 2).reshape(1, cp * n, 512)      # heads s*n + r
    L = l_p.T.reshape(1, cp * n)                             # BH1 layout, H = cp*n
    out, Lm, _ = oracle.merge(O, L, cp, oracle.LSE_BH1, mode)
    o_f, l_f = oracle.attention_full(qb, kb, synth.MLA_SCALE, mode)
    np.testing.assert_allclose(out[0], o_f, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lm[0], l_f, rtol=1e-12)


def test_tiny_config_brute_force():
    """B=3 tokens, 8 local heads, 2 shards of 64 KV rows: merged partials = full attention."""
    q, kv = synth.tiny_attention()
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(kv)
    o_p, l_p = oracle.attention_partials(qb, kb, 2, synth.MLA_SCALE, oracle.BASE_E)
    B, hq = 3, 8
    O = o_p.reshape(B, hq, 2, 512).transpose(0, 2, 1, 3).reshape(B, 2 * hq, 512)
    L = l_p.reshape(B, hq, 2)                                # BHC
    out, Lm, _ = oracle.merge(O, L, 2, oracle.LSE_BHC, oracle.BASE_E)
    o_f, l_f = oracle.attention_full(qb, kb, synth.MLA_SCALE, oracle.BASE_E)
    np.testing.assert_allclose(out.reshape(B * hq, 512), o_f, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lm.reshape(-1), l_f, rtol=1e-13)


def test_sampled_rows_equal_all_rows():
    q, kv = synth.tiny_attention(B=2, hq=4, T=64)
    qb, kb = synth.bf16_bits(q), synth.bf16_bits(kv)
    o_all, l_all = oracle.attention_partials(qb, kb, 2, 0.1, oracle.BASE_E)
    rows = np.array([7, 0, 3])
    o_s, l_s = oracle.attention_partials(qb, kb, 2, 0.1, oracle.BASE_E, rows=rows)
    assert np.array_equal(o_s, o_all[rows]) and np.array_equal(l_s, l_all[rows])
