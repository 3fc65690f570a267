"""Seeded synthetic input generators shared by the HIP path's tests/bench and the oracle.

Only random draws live here: normal samples, bf16 rounding (round to nearest
even, done by torch's dtype conversion), uniform context lengths, and the
mean-shifted key blocks of the 90%-sparsity decode workload.  Nothing here
pools, projects, scores, selects or attends.

Large workloads are drawn on the device with a device generator; small ones
may be drawn on the host.  Either way both sides of a parity check consume
the identical bf16 bits (the oracle gets host copies of the same tensors).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch

from .workloads import DecodeWorkload, PrefillWorkload


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def _normal_bf16(shape, gen, device, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def decode_seqlens(w: DecodeWorkload) -> torch.Tensor:
    """Context length of every sequence (tokens, including the current one), int32 on the host."""
    if w.L is not None:
        return torch.full((w.B,), w.L, dtype=torch.int32)
    lo, hi = w.L_range
    g = _gen(w.seed * 7919 + 17, "cpu")
    return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def decode_capacity(w: DecodeWorkload, seqlens: Optional[torch.Tensor] = None) -> int:
    """Rows allocated per (b, kvh) in the K/V cache: longest context plus growth room, in whole blocks."""
    if seqlens is None:
        seqlens = decode_seqlens(w)
    return round_up(int(seqlens.max()) + w.steps_capacity, w.bs)


def shifted_blocks(w: DecodeWorkload, nc: int, b: int, h: int, layer: int = 0) -> torch.Tensor:
    """Block ids whose keys are mean-shifted for (b, h): round(frac * nc) distinct ids, uniform."""
    n = int(round(w.shifted_frac * nc))
    if n == 0:
        return torch.empty(0, dtype=torch.int64)
    g = _gen(((w.seed * 131 + layer) * 4099 + b) * 257 + h, "cpu")
    return torch.randperm(nc, generator=g)[:n].sort().values


def decode_cache(w: DecodeWorkload, device="cpu", layer: int = 0,
                 seqlens: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """K/V cache [B, Hkv, cap, d] bf16, gate weights [Hkv, dg, d] bf16 and context lengths.

    Rows past a sequence's length hold random values too (they are never read
    as context); the growth rows let a decode loop append tokens.
    """
    if seqlens is None:
        seqlens = decode_seqlens(w)
    cap = decode_capacity(w, seqlens)
    B, H, d = w.B, w.Hkv, w.d
    src_dev = "cpu" if w.fp32_source else device
    gk = _gen(w.seed * 1_000_003 + layer * 101 + 1, src_dev)
    gv = _gen(w.seed * 1_000_003 + layer * 101 + 2, src_dev)
    k = torch.empty((B, H, cap, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, H, cap, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        kf = torch.randn((H, cap, d), generator=gk, device=src_dev, dtype=torch.float32)
        if w.shifted_frac > 0.0:
            nc = int(seqlens[b]) // w.bs
            for h in range(H):
                for blk in shifted_blocks(w, nc, b, h, layer).tolist():
                    kf[h, blk * w.bs:(blk + 1) * w.bs, :] += w.shift
        k[b].copy_(kf.to(torch.bfloat16))
        del kf
        v[b].copy_(torch.randn((H, cap, d), generator=gv, device=src_dev,
                               dtype=torch.float32).to(torch.bfloat16))
    gw = _gen(w.seed * 1_000_003 + layer * 101 + 3, src_dev)
    dg = w.gate_dim
    # Gate projections: variance 1/d_in, the same rule the tiny workload states (N(0, 1/64) at d=64).
    wq = _normal_bf16((H, dg, d), gw, src_dev, std=1.0 / math.sqrt(d)).to(device)
    wk = _normal_bf16((H, dg, d), gw, src_dev, std=1.0 / math.sqrt(d)).to(device)
    return {"k": k, "v": v, "wq": wq, "wk": wk, "seqlens": seqlens.to(device)}


def decode_query(w: DecodeWorkload, step: int = 0, device="cpu") -> torch.Tensor:
    """Fresh query of one decode step: [B, Hq, d] bf16 ~ N(0, 1)."""
    src_dev = "cpu" if w.fp32_source else device
    g = _gen(1000 * w.seed + step, src_dev)
    return _normal_bf16((w.B, w.Hq, w.d), g, src_dev).to(device)


def gate_inputs(B: int, Hq: int, Hkv: int, d: int, dg: int, nb_max: int, seed: int, device="cpu",
                repeat_rows: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of the gate alone: q [B, Hq, d] bf16 ~ N(0, 1), gate weights [Hkv, dg, d] bf16
    ~ N(0, 1/d), and a pooled-key table [B, Hkv, nb_max, d] fp32 ~ N(0, 1/64) (the spread of
    a mean over 64 unit-variance keys).  repeat_rows > 0 copies rows j mod repeat_rows into
    every row j, so that many blocks score exactly alike."""
    g = _gen(seed * 1_000_033 + 5, device)
    out = {"q": _normal_bf16((B, Hq, d), g, device)}
    out["wq"] = _normal_bf16((Hkv, dg, d), g, device, std=1.0 / math.sqrt(d))
    out["wk"] = _normal_bf16((Hkv, dg, d), g, device, std=1.0 / math.sqrt(d))
    kp = torch.randn((B, Hkv, nb_max, d), generator=g, device=device, dtype=torch.float32).mul_(0.125)
    if repeat_rows > 0:
        kp = kp[:, :, torch.arange(nb_max, device=device) % repeat_rows].contiguous()
    out["kpool"] = kp
    return out


def prefill_inputs(w: PrefillWorkload, device="cpu") -> Dict[str, torch.Tensor]:
    """Q, K, V [B, H, L, d] bf16 ~ N(0, 1) and gate weights [H, dg, d] bf16 ~ N(0, 1/d)."""
    shape = (w.B, w.H, w.L, w.d)
    out = {}
    for i, name in enumerate(("q", "k", "v")):
        out[name] = _normal_bf16(shape, _gen(w.seed * 1_000_003 + 11 + i, device), device)
    gw = _gen(w.seed * 1_000_003 + 17, device)
    dg = w.gate_dim
    out["wq"] = _normal_bf16((w.H, dg, w.d), gw, device, std=1.0 / math.sqrt(w.d))
    out["wk"] = _normal_bf16((w.H, dg, w.d), gw, device, std=1.0 / math.sqrt(w.d))
    return out


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bits (what the oracle consumes)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
