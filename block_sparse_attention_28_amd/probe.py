"""Binding of the benchmark's measurement probes (include/seer_probe.h, libseer_probe.so).

Argument marshalling only; the probes measure the part (matrix-core rate, the
decode's read ceiling) and compute nothing of the method.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libseer_probe.so")
_lib = None
_P, _I, _I64 = C.c_void_p, C.c_int, C.c_int64
SIGNATURES = {
    "seer_probe_mfma_bf16": (_I, [_I, _P, _I, _I, _P]),
    "seer_probe_gather_kv": (_I, [_P, _P, _I64, _I64, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
}


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is not built; run __graft_entry__.build() first")
        lib = C.CDLL(_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(name, st):
    if st != 0:
        raise RuntimeError(f"{name} failed ({st})")


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def mfma_bf16(shape: int, sink: torch.Tensor, workgroups: int, iters: int):
    _check("seer_probe_mfma_bf16", load().seer_probe_mfma_bf16(shape, C.c_void_p(sink.data_ptr()), workgroups,
                                                                iters, _stream()))


def gather_kv(k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor, nsel: int, block_size: int,
              num_splits: int, sink: torch.Tensor):
    B, Hkv, cap, d = k.shape
    assert d == 128 and k.stride() == v.stride() and k.stride(3) == 1 and k.stride(2) == d
    assert block_idx.is_contiguous() and block_idx.shape[:2] == (B, Hkv) and block_idx.dtype == torch.int32
    assert sink.numel() >= B * Hkv * num_splits
    _check("seer_probe_gather_kv", load().seer_probe_gather_kv(
        C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()), k.stride(0), k.stride(1), cap,
        C.c_void_p(block_idx.data_ptr()), block_idx.shape[2], nsel, B, Hkv, block_size, num_splits,
        C.c_void_p(sink.data_ptr()), _stream()))
