"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
merge's or the attention's arithmetic.  Both the oracle and the HIP path are
fed from the same host tensors made here.  Everything is generated on the CPU
with ``torch.Generator().manual_seed(seed)``; a GPU copy is the caller's job.

Workloads (shapes and value distributions of the pages' decode geometries;
"N(mu, sigma)" takes sigma as the standard deviation):

* ``tiny_merge``        B=3, H=16, cp=2, D=512; O ~ N(0,1) bf16; base-e LSE ~ U[-5,15],
                        [B, H/cp, cp] layout.  With ``tiny_attention``: q [3, 8, 576],
                        2 shards x 64 KV rows ~ N(0, 0.5), scale 1/sqrt(192).
* ``kimi_merge``        H=64, cp=4 (16 heads/rank), D=512; O ~ N(0,1); base-e LSE ~ U[0,20],
                        [B, H/cp, cp] layout (the 4-GPU Kimi-K2.5 geometry of vLLM PR #48897,
                        latency table).
* ``dsv2_merge``        H=128, cp=8 (16 heads/rank), D=512; O ~ N(0,1); base-2 LSE ~ N(10,4),
                        FlashMLA [B, H, 1] layout (the 8-GPU DeepSeek-V2-236B geometry of
                        sglang PR #40539, Speed Tests).
* ``wide_merge``        cp = 32 or 64 shards of 16 local heads (H = 16 cp), base-e LSE ~ U[0,20], [B, H/cp, cp].
* ``stress_merge``      B=512, in-place [B,64,512] viewed as [B,16,4,512]; LSE ~ U[-30,30] base-e;
                        round(0.1*B*cp) (token, shard) pairs set to -inf (empty shards, all 16 heads
                        of the pair) and their O rows filled with NaN.
* ``mla_decode``        q [B,128,576] ~ N(0,1) bf16, latent KV cache [131072, 576] ~ N(0, 0.5) bf16.
"""
from __future__ import annotations

import math

import numpy as np
import torch

D = 512
D_QK = 576
SEED_BASE = 1000


def gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a CPU bfloat16 tensor as a uint16 numpy array (same shape, contiguous)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, g, mean=0.0, std=1.0) -> torch.Tensor:
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std + mean).to(torch.bfloat16)


def normal_16(shape, g, dtype, mean=0.0, std=1.0) -> torch.Tensor:
    """N(mean, std) drawn in fp32 and rounded to the 16-bit payload type (bf16 or fp16)."""
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std + mean).to(dtype)


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a CPU bf16 or fp16 tensor as a uint16 numpy array (same shape, contiguous)."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def payload_name(t: torch.Tensor) -> str:
    """'bf16' or 'f16': the payload type of a merge input."""
    return "bf16" if t.dtype == torch.bfloat16 else "f16"


def uniform_f32(shape, g, lo, hi) -> torch.Tensor:
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def normal_f32(shape, g, mean, std) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32) * std + mean


class MergeCase:
    """One merge input: the [B, H, D] attention buffer and its LSE tensor."""

    def __init__(self, name, attn, lse, cp, lse_layout, lse_mode, capacity=None):
        self.name = name
        self.attn = attn              # torch bf16 or fp16 [B, H, D] (may be a strided view)
        self.lse = lse                # torch fp32, [B, H/cp, cp] ("bhc") or [B, H, 1] ("bh1")
        self.cp = cp
        self.lse_layout = lse_layout  # "bhc" | "bh1"
        self.lse_mode = lse_mode      # "e" | "2"
        self.capacity = capacity

    @property
    def B(self):
        return self.attn.shape[0]

    @property
    def H(self):
        return self.attn.shape[1]

    @property
    def h_local(self):
        return self.attn.shape[1] // self.cp


def _sfx(dtype):
    return "" if dtype == torch.bfloat16 else " fp16"


def tiny_merge(seed: int = SEED_BASE + 1, dtype=torch.bfloat16) -> MergeCase:
    g = gen(seed)
    B, H, cp = 3, 16, 2
    attn = normal_16((B, H, D), g, dtype)
    lse = uniform_f32((B, H // cp, cp), g, -5.0, 15.0)
    return MergeCase("tiny B=3 H=16 cp=2" + _sfx(dtype), attn, lse, cp, "bhc", "e")


def kimi_merge(B: int, seed: int = SEED_BASE + 2, dtype=torch.bfloat16) -> MergeCase:
    g = gen(seed * 1009 + B)
    H, cp = 64, 4
    attn = normal_16((B, H, D), g, dtype)
    lse = uniform_f32((B, H // cp, cp), g, 0.0, 20.0)
    return MergeCase("kimi-k2.5-like H=64 cp=4 B=%d" % B + _sfx(dtype), attn, lse, cp, "bhc", "e")


def dsv2_merge(B: int, seed: int = SEED_BASE + 3, dtype=torch.bfloat16) -> MergeCase:
    g = gen(seed * 1009 + B)
    H, cp = 128, 8
    attn = normal_16((B, H, D), g, dtype)
    lse = normal_f32((B, H, 1), g, 10.0, 4.0)
    return MergeCase("dsv2-236b-like H=128 cp=8 B=%d" % B + _sfx(dtype), attn, lse, cp, "bh1", "2")


def wide_merge(B: int, cp: int, seed: int = SEED_BASE + 6, dtype=torch.bfloat16) -> MergeCase:
    """More than 16 shards: 16 local heads per rank (the per-rank head count of both geometries above), H = 16 cp,
    base-e LSE ~ U[0, 20] in the [B, H/cp, cp] layout."""
    g = gen(seed * 1009 + B * 131 + cp)
    H = 16 * cp
    attn = normal_16((B, H, D), g, dtype)
    lse = uniform_f32((B, 16, cp), g, 0.0, 20.0)
    return MergeCase("wide H=%d cp=%d B=%d" % (H, cp, B) + _sfx(dtype), attn, lse, cp, "bhc", "e")


def empty_pairs(B: int, cp: int, frac: float, g: torch.Generator) -> torch.Tensor:
    """round(frac*B*cp) distinct (token, shard) pairs, drawn without replacement; bool [B, cp]."""
    n = int(round(frac * B * cp))
    flat = torch.randperm(B * cp, generator=g)[:n]
    mask = torch.zeros(B * cp, dtype=torch.bool)
    mask[flat] = True
    return mask.view(B, cp)


def stress_merge(B: int = 512, seed: int = SEED_BASE + 4, empty_frac: float = 0.1, dtype=torch.bfloat16) -> MergeCase:
    g = gen(seed)
    H, cp = 64, 4
    hl = H // cp
    attn = normal_16((B, H, D), g, dtype)
    lse = uniform_f32((B, hl, cp), g, -30.0, 30.0)
    mask = empty_pairs(B, cp, empty_frac, g)               # [B, cp]
    lse.masked_fill_(mask[:, None, :].expand(B, hl, cp), -math.inf)
    # an empty shard's payload is never written: fill it with NaN so any read shows
    head_mask = mask[:, :, None].expand(B, cp, hl).reshape(B, H)
    attn[head_mask] = float("nan")
    return MergeCase("stress B=%d H=64 cp=4 10%% empty" % B + _sfx(dtype), attn, lse, cp, "bhc", "e", capacity=128)


def tiny_attention(seed: int = SEED_BASE + 1, B: int = 3, hq: int = 8, T: int = 128, dtype=torch.bfloat16):
    g = gen(seed * 7 + 5)
    q = normal_16((B, hq, D_QK), g, dtype)
    kv = normal_16((T, D_QK), g, dtype, 0.0, 0.5)
    return q, kv


def mla_decode(B: int, T: int = 131072, hq: int = 128, seed: int = SEED_BASE + 5, kv_seed=None, dtype=torch.bfloat16):
    """q [B, hq, 576] ~ N(0,1) and one latent KV cache [T, 576] ~ N(0, 0.5), both bf16
    (or fp16).  The cache is drawn from its own seed so every B sees the same cache."""
    gq = gen(seed * 1009 + B)
    q = normal_16((B, hq, D_QK), gq, dtype)
    gk = gen(kv_seed if kv_seed is not None else seed * 1013 + T)
    kv = normal_16((T, D_QK), gk, dtype, 0.0, 0.5)
    return q, kv


MLA_SCALE = 1.0 / math.sqrt(192.0)
