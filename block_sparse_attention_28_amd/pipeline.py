"""One gated sparse decode step, end to end, on preallocated device buffers.

Plumbing only: the plan owns the scratch tensors the C ABI asks for and calls
the five library entry points in order -- gate scores, block selection,
sparse decode (split + merge) -- plus the pooled-key update when blocks
complete.  All arithmetic runs in libseer.so.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import seer


@dataclass
class DecodeShape:
    B: int
    Hq: int
    Hkv: int
    d: int
    bs: int
    budget: int
    nb_max: int
    dg: int

    @property
    def k_max(self) -> int:
        return self.budget // self.bs


class DecodePlan:
    """Scratch buffers and outputs for repeated decode steps of one shape."""

    def __init__(self, shape: DecodeShape, device="cuda", num_splits: int = 0,
                 out_dtype: torch.dtype = torch.bfloat16, gate_scale: float = None,
                 softmax_scale: float = None):
        s = self.shape = shape
        dev = torch.device(device)
        self.gate_scale = 1.0 / math.sqrt(s.dg) if gate_scale is None else gate_scale
        self.softmax_scale = 1.0 / math.sqrt(s.d) if softmax_scale is None else softmax_scale
        self.scores = torch.empty((s.B, s.Hkv, max(s.nb_max, 1)), dtype=torch.float32, device=dev)
        self.block_idx = torch.empty((s.B, s.Hkv, s.k_max), dtype=torch.int32, device=dev)
        self.n_sel = torch.empty((s.B, s.Hkv), dtype=torch.int32, device=dev)
        self.num_splits = seer.seer_sparse_decode_num_splits(s.B, s.Hkv, s.k_max, s.bs, num_splits)
        dws = seer.seer_sparse_decode_workspace_size(s.B, s.Hq, s.Hkv, s.d, s.k_max, s.bs, self.num_splits)
        self.decode_ws = torch.empty((max(dws, 16) + 3) // 4, dtype=torch.float32, device=dev)
        sws = seer.seer_decode_step_workspace_size(s.B, s.Hq, s.Hkv, s.d, s.k_max, s.bs, self.num_splits)
        self.step_ws = torch.empty((max(sws, 16) + 3) // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((s.B, s.Hq, s.d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((s.B, s.Hq), dtype=torch.float32, device=dev)

    def pool(self, k, kpool, upd_b, upd_blk, stream=None):
        seer.seer_pool_k_blocks(k, upd_b, upd_blk, kpool, self.shape.bs, stream=stream)

    def gate(self, q, wq, wk, kpool, seqlens, stream=None):
        seer.seer_gate_scores(q, wq, wk, kpool, seqlens, self.shape.bs, self.gate_scale, self.scores,
                              stream=stream)

    def select(self, seqlens, stream=None):
        seer.seer_select_blocks(self.scores, seqlens, self.shape.bs, self.shape.budget, self.block_idx,
                                self.n_sel, stream=stream)

    def gate_select(self, q, wq, wk, kpool, seqlens, stream=None):
        seer.seer_gate_select(q, wq, wk, kpool, seqlens, self.shape.bs, self.gate_scale, self.shape.budget,
                              self.scores, self.block_idx, self.n_sel, stream=stream)

    def decode(self, q, k, v, seqlens, block_idx=None, n_sel=None, stream=None):
        seer.seer_sparse_decode(q, k, v, seqlens, self.block_idx if block_idx is None else block_idx,
                                self.n_sel if n_sel is None else n_sel, self.shape.bs, self.softmax_scale,
                                self.out, self.lse, self.decode_ws, self.num_splits, stream=stream)

    def step(self, q, k, v, seqlens, kpool, wq, wk, stream=None, mode: str = "calls"):
        """Gate, select and sparse-decode one step; returns (out, lse) views of the plan's buffers.

        mode "calls": seer_gate_scores, seer_select_blocks, seer_sparse_decode; "gate_select":
        seer_gate_select then seer_sparse_decode; "step": seer_decode_step (the gate, then select +
        split decode in one launch, then the merge).  All three give the "calls" results bit for bit."""
        if mode == "step":
            s = self.shape
            seer.seer_decode_step(q, k, v, seqlens, kpool, wq, wk, s.bs, s.budget, self.gate_scale,
                                  self.softmax_scale, self.scores, self.block_idx, self.n_sel, self.out, self.lse,
                                  self.step_ws, self.num_splits, stream=stream)
        elif mode == "calls":
            self.gate(q, wq, wk, kpool, seqlens, stream)
            self.select(seqlens, stream)
            self.decode(q, k, v, seqlens, stream=stream)
        elif mode == "gate_select":
            self.gate_select(q, wq, wk, kpool, seqlens, stream)
            self.decode(q, k, v, seqlens, stream=stream)
        else:
            raise ValueError(f"unknown step mode {mode!r}")
        return self.out, self.lse

    def bind_step(self, q, k, v, seqlens, kpool, wq, wk, mode: str = "calls", stream=None):
        """The launches of one step (as in step()) with their arguments converted once:
        a list of callables, each launching one library call again."""
        s = self.shape
        if mode == "step":
            # seer_decode_step's launches as two calls, so that the last one (select + split decode, merge)
            # can be timed on its own
            return [seer.seer_gate_scores(q, wq, wk, kpool, seqlens, s.bs, self.gate_scale, self.scores,
                                          stream=stream, bind=True),
                    seer.seer_select_sparse_decode(q, k, v, seqlens, self.scores, s.bs, s.budget, self.softmax_scale,
                                                   self.block_idx, self.n_sel, self.out, self.lse, self.step_ws,
                                                   self.num_splits, stream=stream, bind=True)]
        if mode == "calls":
            calls = [seer.seer_gate_scores(q, wq, wk, kpool, seqlens, s.bs, self.gate_scale, self.scores,
                                           stream=stream, bind=True),
                     seer.seer_select_blocks(self.scores, seqlens, s.bs, s.budget, self.block_idx, self.n_sel,
                                             stream=stream, bind=True)]
        elif mode == "gate_select":
            calls = [seer.seer_gate_select(q, wq, wk, kpool, seqlens, s.bs, self.gate_scale, s.budget, self.scores,
                                           self.block_idx, self.n_sel, stream=stream, bind=True)]
        else:
            raise ValueError(f"unknown step mode {mode!r}")
        calls.append(seer.seer_sparse_decode(q, k, v, seqlens, self.block_idx, self.n_sel, s.bs, self.softmax_scale,
                                             self.out, self.lse, self.decode_ws, self.num_splits, stream=stream,
                                             bind=True))
        return calls


def full_pool_lists(seqlens_host: torch.Tensor, bs: int, device="cuda"):
    """(b, j) lists of every complete block of every sequence, for building a pooled cache at once."""
    bl, jl = [], []
    for b, L in enumerate(seqlens_host.tolist()):
        nc = int(L) // bs
        bl.append(torch.full((nc,), b, dtype=torch.int32))
        jl.append(torch.arange(nc, dtype=torch.int32))
    return torch.cat(bl).to(device), torch.cat(jl).to(device)
