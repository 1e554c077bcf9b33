"""The producer's lazy online-softmax rescaling under scores that jump late.

With the seeded inputs (q ~ N(0,1), cache ~ N(0, 0.5), scale 1/sqrt(192)) a
row's scores stay within a few log2 units of the first tile's maximum, so the
kernel's reference maximum never moves after the first tile.  Here keys are
planted in late tiles: cache row t is replaced by alpha * q[b, h], which gives
row (b, h) a score chosen so many log2 units above every score it has seen in
its key range so far -- jumps below the 8-unit margin (the reference stays,
p = 2^(z - m) up to 2^8 is rounded to the 16-bit type) and above it (the
reference moves and the row's accumulators are rescaled), at different tiles
for different rows of one wavefront, so that one rescale step multiplies some
rows by 1 and others by less, and twice in a row for some rows.  Every row is
then checked against the fp64 oracle, on the single-split path, the split path
(partials reduced afterwards) and the variable-length path.
"""
import math

import numpy as np
import pytest
import torch

import context_lse_merge_amd as dcp
import synth
from tests.merge_helpers import announce
from tests.test_gpu_mla import check_end_to_end, check_partials, run_producer
from tests.test_gpu_mla_varlen import check as check_varlen
from tests.test_gpu_mla_varlen import run_varlen

pytestmark = pytest.mark.gpu
LOG2E = 1.0 / math.log(2.0)
KEYS_PER_TILE = 32


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _plant(q, cache, key_rows, row, k, jump):
    """Set cache row key_rows[k] to alpha * q[row] so that row's log2-domain score there lies `jump` above its
    largest score over key_rows[:tile start of k].  Returns the jump actually obtained (after rounding)."""
    qv = q[row].double()
    t0 = (k // KEYS_PER_TILE) * KEYS_PER_TILE
    assert t0 > 0, "plant in a tile after the first"
    prev = cache[key_rows[:t0]].double() @ qv * synth.MLA_SCALE * LOG2E
    m = float(prev.max())
    target = m + jump
    alpha = target / (float(qv @ qv) * synth.MLA_SCALE * LOG2E)
    cache[key_rows[k]] = (alpha * q[row].float()).to(cache.dtype)
    got = float(cache[key_rows[k]].double() @ qv * synth.MLA_SCALE * LOG2E)
    return got - m


# (head, split-local tile, jump in log2 units): heads of one wavefront (0..15) and of another (16..31); heads 2
# and 18 jump twice.  Jumps 5 and 6.5 stay under the 8-unit margin, the others pass it.
PLAN = [(0, 3, 12.0), (1, 5, 7.5), (2, 2, 6.5), (2, 6, 10.0), (3, 7, 30.0), (5, 4, 5.0), (9, 1, 9.0),
        (16, 6, 20.0), (17, 3, 6.5), (18, 2, 9.5), (18, 5, 9.5), (31, 7, 14.0)]


def _plant_plan(q2d, cache, split_rows, b, hq, plan, label):
    """Apply PLAN to token b's rows; split_rows[i] lists the cache rows of the i-th planted split in key order.
    Head h plants in split h % len(split_rows), so a head's two jumps fall in one split."""
    jumps = []
    for i, (h, tile, jump) in enumerate(plan):
        rows = split_rows[h % len(split_rows)]
        k = tile * KEYS_PER_TILE + (7 * i) % KEYS_PER_TILE
        jumps.append(round(_plant(q2d, cache, rows, b * hq + h, k, jump), 2))
    announce("%s: planted jumps %s" % (label, jumps))
    assert min(jumps) < 8.0 < max(jumps)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_single_split_late_jumps(dtype):
    """64 tokens x 128 heads over a 2048-row cache, 4 shards of 512 keys: one split (16 tiles) per shard."""
    B, hq, T, cp = 64, 128, 2048, 4
    assert dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp) == 0
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=8100, dtype=dtype)
    q2d = q.reshape(B * hq, 576)
    shard = T // cp
    for b, s in ((0, 0), (37, 2), (63, 3)):
        base = s * shard
        # tiles of the whole shard: jumps in tiles up to 15
        plan = [(h, 2 * tile + 1, j) for (h, tile, j) in PLAN]
        _plant_plan(q2d, kv, [np.arange(base, base + shard)], b, hq, plan, "single split token %d shard %d" % (b, s))
    o, l = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E)
    worst = check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l)
    announce("single split: all %d rows checked, worst partial row error %.3g of row max" % (B * hq, worst))
    check_end_to_end(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, rows=np.arange(0, B * hq, 7))


def test_split_path_late_jumps():
    """2 tokens x 128 heads over a 16384-row cache: 16 splits of 256 keys (8 tiles) per shard, the splits'
    partials reduced afterwards; jumps late in several splits, and in the last tile of a split."""
    B, hq, T, cp = 2, 128, 16384, 4
    assert dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp) > 0
    q, kv = synth.mla_decode(B, T=T, hq=hq, seed=8200)
    q2d = q.reshape(B * hq, 576)
    shard, split = T // cp, 256
    for b in range(B):
        splits = [np.arange(s * shard + p * split, s * shard + (p + 1) * split) for (s, p) in ((0, 3), (1, 15),
                                                                                              (3, 0), (2, 9))]
        _plant_plan(q2d, kv, splits, b, hq, PLAN, "split path token %d" % b)
    o, l = run_producer(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2)
    worst = check_partials(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l)
    announce("split path: all %d rows checked, worst partial row error %.3g of row max" % (B * hq, worst))
    check_end_to_end(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_2, o, l, rows=np.arange(B * hq))


def test_varlen_late_jumps_interleaved():
    """3 tokens with their own caches and lengths, interleaved ownership: the plan cuts each (token, shard) into
    splits of 256 keys; keys planted late in splits, at the cache rows shard s owns (s, s + cp, ...)."""
    B, hq, T, cp = 3, 128, 12000, 4
    seq = [12000, 9000, 11000]
    g = synth.gen(8300)
    q = synth.normal_16((B, hq, 576), g, torch.bfloat16)
    kv = synth.normal_16((B, T, 576), g, torch.bfloat16, 0.0, 0.5)
    for b in range(B):
        L = seq[b]
        splits = []
        for (s, p) in ((0, 2), (3, 5), (1, 0)):
            owned = np.arange(s, L, cp)
            splits.append(owned[p * 256:(p + 1) * 256])
        _plant_plan(q[b], kv[b], splits, 0, hq, PLAN, "varlen token %d" % b)
    o, l = run_varlen(q, kv, seq, T, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E)
    check_varlen(q, kv, seq, dcp.DCP_KV_INTERLEAVED, cp, dcp.DCP_LSE_BASE_E, o, l)
    announce("varlen: all %d rows checked" % (B * hq))
