"""Thin Python binding of the C ABI in include/seer.h (argument marshalling only).

Each function carries the C name, takes torch tensors that already live on
the GPU, passes their data pointers, strides and the current HIP stream to
libseer.so, and raises ``SeerError`` on a non-zero status.  Every step of the
computation runs in the library's gfx950 kernels; there is no fallback: if
libseer.so is missing or fails to load, the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libseer.so")
_lib = None

SEER_OK = 0
SEER_OUT_BF16 = 0
SEER_OUT_F32 = 1
SEER_KPOOL_F32 = 0
SEER_KPOOL_BF16 = 1
SEER_SELECT_BUDGET, SEER_SELECT_RATIO, SEER_SELECT_THRESHOLD = 0, 1, 2


class SelectPolicy(C.Structure):
    """seer_select_policy: kind (budget / ratio / threshold), ratio_num / ratio_den, threshold."""
    _fields_ = [("kind", C.c_int), ("ratio_num", C.c_int), ("ratio_den", C.c_int), ("threshold", C.c_float)]


def policy(kind: str = "budget", num: int = 1, den: int = 1, tau: float = 0.0) -> SelectPolicy:
    kinds = {"budget": SEER_SELECT_BUDGET, "ratio": SEER_SELECT_RATIO, "threshold": SEER_SELECT_THRESHOLD}
    return SelectPolicy(kinds[kind], int(num), int(den), float(tau))

# name -> (restype, argtypes); mirrors include/seer.h
_P, _I, _I64, _F, _SZ = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
SIGNATURES = {
    "seer_status_string": (C.c_char_p, [_I]),
    "seer_version": (_I, []),
    "seer_pool_k_blocks": (_I, [_P, _I64, _I64, _I64, _I, _I, _I, _I, _I, _P, _P, _I, _P, _I, _P]),
    "seer_pool_k_blocks_ex": (_I, [_P, _I64, _I64, _I64, _I, _I, _I, _I, _I, _P, _P, _I, _P, _I, _I, _P]),
    "seer_gate_scores": (_I, [_P, _I64, _I64, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P]),
    "seer_select_blocks": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "seer_select_blocks_ex": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "seer_gate_select_ex": (_I, [_P, _I64, _I64, _P, _P, _I, _P, _I, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                                 _P, _P]),
    "seer_gate_select": (_I, [_P, _I64, _I64, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P]),
    "seer_sparse_decode_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "seer_sparse_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "seer_sparse_decode": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _I, _I, _I, _I, _I,
                                _I, _F, _I, _P, _SZ, _P, _I, _P, _P]),
    "seer_sparse_decode_noalloc": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _I, _I, _I, _I,
                                        _I, _I, _F, _I, _P, _I, _P, _P]),
    "seer_gate_select_heads": (_I, [_P, _I64, _I64, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                                    _P]),
    "seer_sparse_decode_heads_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "seer_sparse_decode_heads": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _I, _I, _I, _I,
                                      _I, _I, _I, _F, _I, _P, _SZ, _P, _I, _P, _P]),
    "seer_decode_block_mass_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "seer_decode_block_mass": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _I, _I, _I, _I, _I, _F, _I,
                                    _I, _P, _SZ, _P, _I, _P, _P, _P]),
    "seer_prefill_block_mass": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P]),
    "seer_decode_step_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "seer_decode_step": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _I, _F, _P, _I, _I, _I, _I,
                              _I, _I, _I, _F, _I, _P, _P, _P, _P, _SZ, _P, _I, _P, _P]),
    "seer_select_sparse_decode": (_I, [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _I, _F, _I, _P, _P, _P, _SZ, _P, _I, _P, _P]),
    "seer_block_sparse_prefill_kmax_row": (_I, [_I, _I, _I, _I]),
    "seer_block_sparse_prefill_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "seer_block_sparse_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _F, _I, _I, _P, _P, _I, _I, _F,
                                       _P, _SZ, _P, _P, _P]),
}


class SeerError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libseer.so (built in-tree by block_sparse_attention_28_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python -m block_sparse_attention_28_amd.build) first")
        lib = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().seer_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("seer kernels take device tensors")
    return C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


_BYREF = type(C.byref(C.c_int(0)))


class Bound:
    """One library call with its arguments converted to C values once; calling the
    object launches it again (for tight step loops where the marshalling would
    otherwise cost more host time than the launch)."""
    __slots__ = ("name", "fn", "args")

    def __init__(self, name: str, args):
        self.name = name
        self.fn = getattr(load(), name)
        types = SIGNATURES[name][1]
        keep = (C._SimpleCData, _BYREF)
        self.args = tuple(a if a is None or isinstance(a, keep) else t(a) for t, a in zip(types, args))

    def __call__(self):
        st = self.fn(*self.args)
        if st != SEER_OK:
            raise SeerError(self.name, st)


def _call(name: str, *args, bind: bool = False):
    if bind:
        return Bound(name, args)
    st = getattr(load(), name)(*args)
    if st != SEER_OK:
        raise SeerError(name, st)


def _bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected bfloat16, got {t.dtype}")
    return t


def seer_pool_k_blocks(k, upd_b, upd_blk, kpool, block_size: int, stream=None, bind: bool = False):
    """kpool[b, :, j] = mean of block j of k[b] for each listed (b, j).  k [B, Hkv, cap, d] bf16."""
    _bits(k)
    B, Hkv, cap, d = k.shape
    assert kpool.dtype == torch.float32 and kpool.is_contiguous() and kpool.shape[:2] == (B, Hkv)
    assert upd_b.dtype == torch.int32 and upd_blk.dtype == torch.int32 and upd_b.numel() == upd_blk.numel()
    return _call(
        "seer_pool_k_blocks", _ptr(k), k.stride(0), k.stride(1), k.stride(2), B, Hkv, d, block_size, cap,
        _ptr(upd_b), _ptr(upd_blk), upd_b.numel(), _ptr(kpool), kpool.shape[2], _stream(stream), bind=bind)


def seer_pool_k_blocks_ex(k, upd_b, upd_blk, kpool, block_size: int, stream=None, bind: bool = False):
    """seer_pool_k_blocks into an fp32 or bf16 table (its dtype decides)."""
    _bits(k)
    B, Hkv, cap, d = k.shape
    assert kpool.is_contiguous() and kpool.shape[:2] == (B, Hkv)
    assert upd_b.dtype == torch.int32 and upd_blk.dtype == torch.int32 and upd_b.numel() == upd_blk.numel()
    return _call(
        "seer_pool_k_blocks_ex", _ptr(k), k.stride(0), k.stride(1), k.stride(2), B, Hkv, d, block_size, cap,
        _ptr(upd_b), _ptr(upd_blk), upd_b.numel(), _ptr(kpool), _kpool_dtype(kpool), kpool.shape[2],
        _stream(stream), bind=bind)


def seer_gate_scores(q, wq, wk, kpool, seqlens, block_size: int, gate_scale: float, scores, stream=None,
                     bind: bool = False):
    """scores [B, Hkv, nb_max] fp32 from q [B, Hq, d], wq/wk [Hkv, dg, d], kpool [B, Hkv, nb_max, d]."""
    _bits(q), _bits(wq), _bits(wk)
    B, Hq, d = q.shape
    Hkv, dg, _ = wq.shape
    assert wq.is_contiguous() and wk.is_contiguous() and kpool.is_contiguous() and scores.is_contiguous()
    return _call(
        "seer_gate_scores", _ptr(q), q.stride(0), q.stride(1), _ptr(wq), _ptr(wk), dg, _ptr(kpool), kpool.shape[2],
        _ptr(seqlens), B, Hq, Hkv, d, block_size, float(gate_scale), _ptr(scores), _stream(stream), bind=bind)


def seer_select_blocks(scores, seqlens, block_size: int, budget_tokens: int, block_idx, n_sel, stream=None,
                       bind: bool = False):
    """block_idx [B, H, budget // bs] int32 (ascending, -1 padded), n_sel [B, H] int32."""
    B, H, nb_max = scores.shape
    assert scores.is_contiguous() and n_sel.is_contiguous()
    return _call(
        "seer_select_blocks", _ptr(scores), _ptr(seqlens), B, H, nb_max, block_size, budget_tokens,
        _ptr(block_idx) if block_idx is not None and block_idx.numel() else None, _ptr(n_sel), _stream(stream),
        bind=bind)


def seer_gate_select(q, wq, wk, kpool, seqlens, block_size: int, gate_scale: float, budget_tokens: int, scores,
                     block_idx, n_sel, stream=None, bind: bool = False):
    """seer_gate_scores then seer_select_blocks on those scores, in one launch where the shape allows."""
    _bits(q), _bits(wq), _bits(wk)
    B, Hq, d = q.shape
    Hkv, dg, _ = wq.shape
    assert wq.is_contiguous() and wk.is_contiguous() and kpool.is_contiguous() and scores.is_contiguous()
    assert n_sel.is_contiguous()
    return _call(
        "seer_gate_select", _ptr(q), q.stride(0), q.stride(1), _ptr(wq), _ptr(wk), dg, _ptr(kpool), kpool.shape[2],
        _ptr(seqlens), B, Hq, Hkv, d, block_size, float(gate_scale), budget_tokens, _ptr(scores),
        _ptr(block_idx) if block_idx is not None and block_idx.numel() else None, _ptr(n_sel), _stream(stream),
        bind=bind)


def _kpool_dtype(kpool) -> int:
    if kpool.dtype == torch.float32:
        return SEER_KPOOL_F32
    if kpool.dtype == torch.bfloat16:
        return SEER_KPOOL_BF16
    raise TypeError(f"pooled keys must be float32 or bfloat16, got {kpool.dtype}")


def seer_select_blocks_ex(scores, seqlens, block_size: int, k_max: int, pol: Optional[SelectPolicy], block_idx,
                          n_sel, stream=None, bind: bool = False):
    """Selection by a policy (budget / ratio / threshold); block_idx [B, H, k_max]."""
    B, H, nb_max = scores.shape
    assert scores.is_contiguous() and n_sel.is_contiguous()
    return _call(
        "seer_select_blocks_ex", _ptr(scores), _ptr(seqlens), B, H, nb_max, block_size, int(k_max),
        C.byref(pol) if pol is not None else None, _ptr(block_idx) if k_max else None, _ptr(n_sel),
        _stream(stream), bind=bind)


def seer_gate_select_ex(q, wq, wk, kpool, seqlens, block_size: int, gate_scale: float, k_max: int,
                        pol: Optional[SelectPolicy], scores, block_idx, n_sel, stream=None, bind: bool = False):
    """seer_gate_select with a selection policy and an fp32 or bf16 pooled-key table."""
    _bits(q), _bits(wq), _bits(wk)
    B, Hq, d = q.shape
    Hkv, dg, _ = wq.shape
    assert wq.is_contiguous() and wk.is_contiguous() and kpool.is_contiguous() and scores.is_contiguous()
    assert n_sel.is_contiguous()
    return _call(
        "seer_gate_select_ex", _ptr(q), q.stride(0), q.stride(1), _ptr(wq), _ptr(wk), dg, _ptr(kpool),
        _kpool_dtype(kpool), kpool.shape[2], _ptr(seqlens), B, Hq, Hkv, d, block_size, float(gate_scale), int(k_max),
        C.byref(pol) if pol is not None else None, _ptr(scores), _ptr(block_idx) if k_max else None, _ptr(n_sel),
        _stream(stream), bind=bind)


def seer_sparse_decode_num_splits(B: int, Hkv: int, k_max: int, block_size: int, num_splits: int = 0) -> int:
    return load().seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits)


def seer_sparse_decode_workspace_size(B: int, Hq: int, Hkv: int, d: int, k_max: int, block_size: int,
                                      num_splits: int = 0) -> int:
    return load().seer_sparse_decode_workspace_size(B, Hq, Hkv, d, k_max, block_size, num_splits)


def seer_sparse_decode(q, k, v, seqlens, block_idx, n_sel, block_size: int, softmax_scale: float, out,
                       lse=None, workspace=None, num_splits: int = 0, stream=None, bind: bool = False):
    """out [B, Hq, d] (bf16 or fp32) = attention of q over the kept blocks + tail of k/v [B, Hkv, cap, d]."""
    _bits(q), _bits(k), _bits(v)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert k.stride() == v.stride() and out.is_contiguous()
    k_max = block_idx.shape[2] if block_idx is not None else 0
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _call(
        "seer_sparse_decode", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), cap, _ptr(seqlens), _ptr(block_idx) if k_max else None, _ptr(n_sel), k_max, B, Hq, Hkv, d,
        block_size, float(softmax_scale), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), out_dtype,
        _ptr(lse), _stream(stream), bind=bind)


def seer_sparse_decode_noalloc(q, k, v, seqlens, block_idx, n_sel, block_size: int, softmax_scale: float, out,
                               lse=None, num_splits: int = 0, stream=None, bind: bool = False):
    """seer_sparse_decode with its split partials in the library's static device scratch (no workspace)."""
    _bits(q), _bits(k), _bits(v)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert k.stride() == v.stride() and out.is_contiguous()
    k_max = block_idx.shape[2] if block_idx is not None else 0
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    return _call(
        "seer_sparse_decode_noalloc", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0),
        k.stride(1), k.stride(2), cap, _ptr(seqlens), _ptr(block_idx) if k_max else None, _ptr(n_sel), k_max, B, Hq,
        Hkv, d, block_size, float(softmax_scale), int(num_splits), _ptr(out), out_dtype, _ptr(lse), _stream(stream),
        bind=bind)


def seer_gate_select_heads(q, wq, wk, kpool, seqlens, block_size: int, gate_scale: float, budget_tokens: int,
                           scores, block_idx, n_sel, stream=None, bind: bool = False):
    """Per-query-head gate scores [B, Hq, nb_max] and selections [B, Hq, budget // bs]."""
    _bits(q), _bits(wq), _bits(wk)
    B, Hq, d = q.shape
    Hkv, dg, _ = wq.shape
    assert wq.is_contiguous() and wk.is_contiguous() and kpool.is_contiguous() and scores.is_contiguous()
    assert n_sel.is_contiguous() and scores.shape == (B, Hq, kpool.shape[2])
    return _call(
        "seer_gate_select_heads", _ptr(q), q.stride(0), q.stride(1), _ptr(wq), _ptr(wk), dg, _ptr(kpool),
        kpool.shape[2], _ptr(seqlens), B, Hq, Hkv, d, block_size, float(gate_scale), budget_tokens, _ptr(scores),
        _ptr(block_idx) if block_idx is not None and block_idx.numel() else None, _ptr(n_sel), _stream(stream),
        bind=bind)


def seer_sparse_decode_heads_workspace_size(B: int, Hq: int, Hkv: int, d: int, k_max: int, nb_max: int,
                                            block_size: int, num_splits: int = 0) -> int:
    return load().seer_sparse_decode_heads_workspace_size(B, Hq, Hkv, d, k_max, nb_max, block_size, num_splits)


def seer_sparse_decode_heads(q, k, v, seqlens, block_idx, n_sel, nb_max: int, block_size: int,
                             softmax_scale: float, out, lse=None, workspace=None, num_splits: int = 0, stream=None,
                             bind: bool = False):
    """Sparse decode over per-query-head block sets (block_idx [B, Hq, k_max]): the union read once per group."""
    _bits(q), _bits(k), _bits(v)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert k.stride() == v.stride() and out.is_contiguous() and block_idx.is_contiguous()
    k_max = block_idx.shape[2]
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _call(
        "seer_sparse_decode_heads", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), cap, _ptr(seqlens), _ptr(block_idx) if k_max else None, _ptr(n_sel), k_max, int(nb_max), B,
        Hq, Hkv, d, block_size, float(softmax_scale), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out),
        out_dtype, _ptr(lse), _stream(stream), bind=bind)


def seer_decode_block_mass_workspace_size(B: int, Hq: int, Hkv: int, d: int, nb_max: int, block_size: int,
                                          num_splits: int = 0) -> int:
    return load().seer_decode_block_mass_workspace_size(B, Hq, Hkv, d, nb_max, block_size, num_splits)


def seer_decode_block_mass(q, k, v, seqlens, block_size: int, softmax_scale: float, mass, out, lse=None,
                           workspace=None, num_splits: int = 0, stream=None, bind: bool = False):
    """Dense attention of q over the whole context of k/v [B, Hkv, cap, d] into out, and the group-mean
    attention mass of every block into mass [B, Hkv, nb_max + 1] (last slot: the tail)."""
    _bits(q), _bits(k), _bits(v)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert k.stride() == v.stride() and out.is_contiguous() and mass.is_contiguous()
    assert mass.dtype == torch.float32 and mass.shape[:2] == (B, Hkv)
    nb_max = mass.shape[2] - 1
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    return _call(
        "seer_decode_block_mass", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), cap, _ptr(seqlens), B, Hq, Hkv, d, block_size, float(softmax_scale), nb_max, int(num_splits),
        _ptr(workspace), ws_bytes, _ptr(out), out_dtype, _ptr(lse), _ptr(mass), _stream(stream), bind=bind)


def seer_block_sparse_prefill_kmax_row(L: int, block_size: int, keep_num: int, keep_den: int) -> int:
    return load().seer_block_sparse_prefill_kmax_row(L, block_size, keep_num, keep_den)


def seer_block_sparse_prefill_workspace_size(B: int, H: int, L: int, d: int, block_size: int, dg: int) -> int:
    return load().seer_block_sparse_prefill_workspace_size(B, H, L, d, block_size, dg)


def seer_block_sparse_prefill(q, k, v, block_size: int, wq, wk, gate_scale: float, keep_num: int, keep_den: int,
                              kv_blocks, kv_count, softmax_scale: float, out, lse=None, workspace=None,
                              use_given_blocks: bool = False, stream=None):
    """Block-sparse causal prefill of q, k, v [B, H, L, d] bf16 into out; kv_blocks [B, H, nb, kmax_row]."""
    _bits(q), _bits(k), _bits(v), _bits(out)
    B, H, L, d = q.shape
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous() and out.is_contiguous()
    assert kv_blocks.dtype == torch.int32 and kv_count.dtype == torch.int32 and kv_blocks.is_contiguous()
    dg = wq.shape[1] if wq is not None else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("seer_block_sparse_prefill", _ptr(q), _ptr(k), _ptr(v), B, H, L, d, block_size, _ptr(wq), _ptr(wk), dg,
          float(gate_scale), keep_num, keep_den, _ptr(kv_blocks), _ptr(kv_count), kv_blocks.shape[-1],
          1 if use_given_blocks else 0, float(softmax_scale), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
          _stream(stream))


def seer_prefill_block_mass(q, k, v, block_size: int, softmax_scale: float, out, mass, lse=None, stream=None,
                            bind: bool = False):
    """Dense causal attention of q, k, v [B, H, L, d] into out, and mass [B, H, nb, nb]: per query block the
    mean attention mass of every key block."""
    _bits(q), _bits(k), _bits(v), _bits(out)
    B, H, L, d = q.shape
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous() and out.is_contiguous()
    assert mass.dtype == torch.float32 and mass.is_contiguous()
    return _call(
        "seer_prefill_block_mass", _ptr(q), _ptr(k), _ptr(v), B, H, L, d, block_size, float(softmax_scale),
        _ptr(out), _ptr(lse), _ptr(mass), _stream(stream), bind=bind)


def seer_decode_step_workspace_size(B: int, Hq: int, Hkv: int, d: int, k_max: int, block_size: int,
                                    num_splits: int = 0) -> int:
    return load().seer_decode_step_workspace_size(B, Hq, Hkv, d, k_max, block_size, num_splits)


def seer_decode_step(q, k, v, seqlens, kpool, wq, wk, block_size: int, budget_tokens: int, gate_scale: float,
                     softmax_scale: float, scores, block_idx, n_sel, out, lse=None, workspace=None,
                     num_splits: int = 0, stream=None, bind: bool = False):
    """Gate + select + sparse decode in three launches: the gate, select + split decode, the merge
    (same results as the three separate calls)."""
    _bits(q), _bits(k), _bits(v), _bits(wq), _bits(wk)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    dg = wq.shape[1]
    assert k.stride() == v.stride() and out.is_contiguous() and kpool.is_contiguous() and scores.is_contiguous()
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    k_max = budget_tokens // block_size
    return _call(
        "seer_decode_step", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), cap, _ptr(seqlens), _ptr(wq), _ptr(wk), dg, float(gate_scale), _ptr(kpool), kpool.shape[2], B,
        Hq, Hkv, d, block_size, int(budget_tokens), float(softmax_scale), int(num_splits), _ptr(scores),
        _ptr(block_idx) if k_max else None, _ptr(n_sel), _ptr(workspace), ws_bytes, _ptr(out), out_dtype, _ptr(lse),
        _stream(stream), bind=bind)


def seer_select_sparse_decode(q, k, v, seqlens, scores, block_size: int, budget_tokens: int, softmax_scale: float,
                              block_idx, n_sel, out, lse=None, workspace=None, num_splits: int = 0, stream=None,
                              bind: bool = False):
    """From given gate scores [B, Hkv, nb_max]: the selection inside the decode kernel, then the merge
    (seer_decode_step's last two launches; same results as seer_select_blocks + seer_sparse_decode)."""
    _bits(q), _bits(k), _bits(v)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert k.stride() == v.stride() and out.is_contiguous() and scores.is_contiguous()
    out_dtype = SEER_OUT_F32 if out.dtype == torch.float32 else SEER_OUT_BF16
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    k_max = budget_tokens // block_size
    return _call(
        "seer_select_sparse_decode", _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), cap, _ptr(seqlens), _ptr(scores), scores.shape[2], B, Hq, Hkv, d, block_size,
        int(budget_tokens), float(softmax_scale), int(num_splits), _ptr(block_idx) if k_max else None, _ptr(n_sel),
        _ptr(workspace) if workspace is not None else None, ws_bytes, _ptr(out), out_dtype, _ptr(lse),
        _stream(stream), bind=bind)
