"""Synthetic workloads for gated block-sparse decode and block-sparse prefill.

Each workload is named for what it is and carries its sizes.  The shapes
follow the regime the SeerAttention-R abstract describes for decoding (a 4K
token budget, 64- or 128-token blocks, long contexts at about 90% sparsity)
and the regime the SeerAttention (v2) abstract describes for prefill (32k
context, 90% sparsity).  Neither page prints tensor shapes, so batch, head
counts, head_dim and value distributions are choices stated here.

This module holds sizes only: no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int                      # sequences in the batch
    Hq: int                     # query heads
    Hkv: int                    # KV heads (GQA group size G = Hq // Hkv)
    d: int                      # head_dim
    bs: int                     # KV block size in tokens
    budget: int                 # token budget; k = budget // bs selected blocks
    seed: int
    L: Optional[int] = None     # uniform context length (tokens, incl. current)
    L_range: Optional[Tuple[int, int]] = None  # ragged: L_b ~ U[lo, hi] inclusive
    dg: int = 0                 # gate projection width (0 -> d)
    shifted_frac: float = 0.0   # fraction of blocks per (b, kvh) whose keys get +shift
    shift: float = 0.0
    fp32_source: bool = False   # draw Q/K/V in fp32 on the host before bf16 rounding
    steps_capacity: int = 0     # extra cache rows so L can grow while decoding

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def gate_dim(self) -> int:
        return self.dg or self.d

    @property
    def k_max(self) -> int:
        return self.budget // self.bs


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    H: int                      # heads (MHA: query heads == KV heads)
    L: int
    d: int
    bs: int                     # square block size (query blocks x key blocks)
    keep_num: int               # keep ceil((i+1) * num / den) causal blocks in row i
    keep_den: int
    seed: int
    dg: int = 0

    @property
    def gate_dim(self) -> int:
        return self.dg or self.d


TINY_DECODE = DecodeWorkload(
    name="tiny_decode_b1_g4_d64_l1024_bs64_k4", B=1, Hq=4, Hkv=1, d=64, bs=64,
    budget=256, seed=0, L=1024, fp32_source=True)

DECODE_L32K = DecodeWorkload(
    name="decode_b8_h32x8_d128_l32768_bs64_budget4096", B=8, Hq=32, Hkv=8, d=128,
    bs=64, budget=4096, seed=1, L=32768)

# Headline: 51 of 512 blocks per (b, kvh) -> 90.04% sparsity.
DECODE_L64K_S90 = DecodeWorkload(
    name="decode_b16_h32x8_d128_l65536_bs128_k51", B=16, Hq=32, Hkv=8, d=128,
    bs=128, budget=6553, seed=2, L=65536, shifted_frac=0.05, shift=2.0)

RAGGED_DECODE = DecodeWorkload(
    name="ragged_decode_b32_h64x8_d128_l8k-128k_bs64_budget4096", B=32, Hq=64,
    Hkv=8, d=128, bs=64, budget=4096, seed=3, L_range=(8192, 131072),
    steps_capacity=64)

PREFILL_L32K = PrefillWorkload(
    name="prefill_b1_h32_d128_l32768_bs64_keep10pct", B=1, H=32, L=32768, d=128,
    bs=64, keep_num=1, keep_den=10, seed=4)

DECODE_WORKLOADS = {w.name: w for w in (TINY_DECODE, DECODE_L32K, DECODE_L64K_S90, RAGGED_DECODE)}
PREFILL_WORKLOADS = {w.name: w for w in (PREFILL_L32K,)}
