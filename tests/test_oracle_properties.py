"""Hypothesis properties of the fp64 oracle merge over random geometries.

Each drawn case -- tokens, local heads, shard count, head size, LSE base and
layout, LSE spread and a random set of empty shards (LSE = -inf, payload
NaN) -- is checked against scipy's softmax / logsumexp applied to the same
numbers, with the head mapping h = s*(H/cp) + j of the [B,H/cp,cp,D] view
(sglang PR #40539, Modifications) and the empty-shard rules (vLLM PR #48897,
port commit: -inf marks an empty shard whose payload is never read; sglang
PR #32851, commit log: an all-empty row gives 0).  The oracle must also be
invariant to a common LSE shift and to a permutation of the shards.
"""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import logsumexp, softmax

import oracle

LN2 = math.log(2.0)


@st.composite
def merge_cases(draw):
    B = draw(st.integers(1, 4))
    hl = draw(st.integers(1, 5))
    cp = draw(st.integers(1, 9))
    D = draw(st.sampled_from([1, 8, 24]))
    mode = draw(st.sampled_from([oracle.BASE_E, oracle.BASE_2]))
    layout = draw(st.sampled_from([oracle.LSE_BHC, oracle.LSE_BH1]))
    spread = draw(st.sampled_from([0.0, 1.0, 30.0, 80.0]))
    centre = draw(st.floats(-50, 50))
    p_empty = draw(st.sampled_from([0.0, 0.2, 0.6, 1.0]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return B, hl, cp, D, mode, layout, spread, centre, p_empty, seed


def _draw_arrays(B, hl, cp, D, spread, centre, p_empty, seed):
    rng = np.random.default_rng(seed)
    O = rng.standard_normal((B, hl * cp, D))
    lse = centre + spread * rng.uniform(-1, 1, size=(B, hl, cp))
    empty = rng.random((B, hl, cp)) < p_empty
    lse[empty] = -np.inf
    # an empty shard's payload is stale: make it NaN so any read shows
    O4 = O.reshape(B, cp, hl, D)
    O4[empty.transpose(0, 2, 1)] = np.nan
    return O4.reshape(B, hl * cp, D), lse, empty


def _as_layout(lse_bhc, layout):
    B, hl, cp = lse_bhc.shape
    return lse_bhc if layout == oracle.LSE_BHC else np.ascontiguousarray(lse_bhc.transpose(0, 2, 1)).reshape(B, hl * cp)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(merge_cases())
def test_oracle_merge_equals_softmax_weighting(case):
    B, hl, cp, D, mode, layout, spread, centre, p_empty, seed = case
    O, lse, empty = _draw_arrays(B, hl, cp, D, spread, centre, p_empty, seed)
    out, L, A = oracle.merge(O, _as_layout(lse, layout), cp, layout, mode)
    Os = O.reshape(B, cp, hl, D).transpose(0, 2, 1, 3)      # [B, hl, cp, D]
    nat = lse if mode == oracle.BASE_E else lse * LN2
    for b in range(B):
        for j in range(hl):
            used = ~empty[b, j]
            if not used.any():
                assert np.all(out[b, j] == 0) and not np.signbit(out[b, j]).any()
                assert np.isneginf(L[b, j])
                continue
            p = softmax(nat[b, j, used])
            ref = p @ Os[b, j, used]
            np.testing.assert_allclose(out[b, j], ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(A[b, j], p @ np.abs(Os[b, j, used]), rtol=1e-11, atol=1e-12)
            refL = logsumexp(nat[b, j, used]) / (1.0 if mode == oracle.BASE_E else LN2)
            assert abs(L[b, j] - refL) <= 1e-12 * max(abs(refL), 1.0)


@settings(max_examples=80, deadline=None)
@given(merge_cases(), st.integers(-40, 40))
def test_oracle_shift_and_shard_permutation_invariance(case, shift):
    B, hl, cp, D, mode, layout, spread, centre, p_empty, seed = case
    O, lse, empty = _draw_arrays(B, hl, cp, D, spread, centre, 0.0, seed)
    out, L, _ = oracle.merge(O, lse, cp, oracle.LSE_BHC, mode)
    # a common shift by an integer moves L by exactly that amount and leaves out unchanged
    out2, L2, _ = oracle.merge(O, lse + shift, cp, oracle.LSE_BHC, mode)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L + shift, rtol=1e-12, atol=1e-12)
    # permuting the shards (payload heads and LSE together) changes nothing
    perm = np.random.default_rng(seed).permutation(cp)
    Op = O.reshape(B, cp, hl, D)[:, perm].reshape(B, cp * hl, D)
    out3, L3, _ = oracle.merge(Op, lse[:, :, perm], cp, oracle.LSE_BHC, mode)
    np.testing.assert_allclose(out3, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L3, L, rtol=1e-13, atol=1e-13)
