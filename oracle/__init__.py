"""fp64 CPU oracle of gated block-sparse decode and block-sparse prefill.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  The arithmetic
lives in plain C (``seer_oracle.c``); this module only compiles it with gcc,
loads it with ctypes and marshals numpy arrays.  bf16 inputs are passed as
their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "seer_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libseer_oracle.so")
_lib = None


def build(quiet: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no fast-math) into oracle/libseer_oracle.so."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "seer_oracle.h"))):
        build()
    _lib = _bind(_LIB_PATH)
    return _lib


def _bind(path: str):
    """Load an oracle build at ``path`` and declare its C signatures."""
    lib = C.CDLL(path)
    P, I, I64, D = C.c_void_p, C.c_int, C.c_int64, C.c_double
    sig = {
        "so_bf16_to_f64": (D, [C.c_uint16]),
        "so_max_threads": (I, []),
        "so_pool_k": (I, [P, I64, I, I, I, P]),
        "so_gate_scores": (I, [P, I64, I, I, P, P, I, P, I, D, P, P]),
        "so_select_blocks": (I, [P, I, I, P]),
        "so_select_policy": (I, [P, I, I, I, I, I, D, P]),
        "so_sparse_attention": (I, [P, I64, I, I, P, P, I64, I, I, P, I, D, P, P, P]),
        "so_decode_block_mass": (I, [P, I64, I, I, P, P, I64, I, I, D, P, P, P]),
        "so_pool_cache": (I, [P, I64, I64, I64, P, I, I, I, I, I, P]),
        "so_decode_step": (I, [P, I64, I64, P, P, I64, I64, I64, P, I, I, I, I, I, I,
                               P, P, I, D, P, I, D, P, P, P, P, P]),
        "so_decode_step_per_head": (I, [P, I64, I64, P, P, I64, I64, I64, P, I, I, I, I, I, I,
                                        P, P, I, D, P, I, D, P, P, P, P, P]),
        "so_prefill_block_mass": (I, [P, P, I64, I, I, I, D, I, I, P]),
        "so_prefill_gate": (I, [P, P, I64, I, I, I, P, P, I, D, I, I, P, P, P, I]),
        "so_prefill_attention": (I, [P, P, P, I64, I, I, I, P, P, I, D, I, I, P, P]),
        "so_prefill": (I, [P, P, P, I, I, I, I, I, P, P, I, D, I, I, P, P, I, D, I, I, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc < 0:
        raise ValueError(f"oracle {what}: precondition violated (rc={rc})")


def max_threads() -> int:
    return _load().so_max_threads()


def bf16_to_f64(bits: int) -> float:
    return _load().so_bf16_to_f64(int(bits))


def pool_k(k, bs: int) -> np.ndarray:
    """Mean of each complete bs-token block of one head's keys k [L, d] -> [L // bs, d]."""
    k = _u16(k)
    L, d = k.shape
    out = np.zeros((L // bs, d), dtype=np.float64)
    _check(_load().so_pool_k(_p(k), d, L, d, bs, _p(out)), "pool_k")
    return out


def gate_scores(q, wq, wk, kpool, gate_scale: float):
    """Literal gate of one KV head: q [G, d] group rows, wq/wk [dg, d], kpool [nc, d] fp64.

    Returns (s_head [G, nc], S [nc]) where S is the group mean."""
    q, wq, wk, kpool = _u16(q), _u16(wq), _u16(wk), _f64(kpool)
    G, d = q.shape
    dg = wq.shape[0]
    nc = kpool.shape[0]
    s_head = np.zeros((G, nc), dtype=np.float64)
    S = np.zeros((nc,), dtype=np.float64)
    _check(_load().so_gate_scores(_p(q), d, G, d, _p(wq), _p(wk), dg, _p(kpool), nc,
                                  float(gate_scale), _p(s_head), _p(S)), "gate_scores")
    return s_head, S


def select_blocks(S, k: int) -> np.ndarray:
    """Ascending ids of the min(k, nc) best blocks by (score desc, id asc)."""
    S = _f64(S)
    idx = np.full((max(k, 1),), -1, dtype=np.int32)
    n = _load().so_select_blocks(_p(S), S.shape[0], int(k), _p(idx))
    _check(n, "select_blocks")
    return idx[:n].copy()


POLICY_BUDGET, POLICY_RATIO, POLICY_THRESHOLD = 0, 1, 2


def select_policy(S, policy: int, k_max: int, num: int = 1, den: int = 1, tau: float = 0.0) -> np.ndarray:
    """Ascending ids kept by a selection policy (budget / ratio / threshold) over scores S [nc]."""
    S = _f64(S)
    idx = np.full((max(k_max, 1),), -1, dtype=np.int32)
    n = _load().so_select_policy(_p(S), S.shape[0], int(policy), int(k_max), int(num), int(den), float(tau), _p(idx))
    _check(n, "select_policy")
    return idx[:n].copy()


def sparse_attention(q, k, v, bs: int, idx, scale: float, L: Optional[int] = None,
                     want_weights: bool = False):
    """Attention of q [G, d] over kept blocks idx plus the tail of k/v [>=L, d].

    Returns (out [G, d], lse [G], weights [G, L] or None)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    idx = _i32(idx)
    G, d = q.shape
    if L is None:
        L = k.shape[0]
    assert k.shape[0] >= L and v.shape == k.shape
    out = np.zeros((G, d), dtype=np.float64)
    lse = np.zeros((G,), dtype=np.float64)
    w = np.zeros((G, L), dtype=np.float64) if want_weights else None
    _check(_load().so_sparse_attention(_p(q), d, G, d, _p(k), _p(v), d, L, bs, _p(idx), idx.shape[0],
                                       float(scale), _p(out), _p(lse), _p(w)), "sparse_attention")
    return out, lse, w


def decode_block_mass(q, k, v, bs: int, scale: float, L: Optional[int] = None):
    """Ground truth of one KV head's decode: dense attention of q [G, d] over k/v [>=L, d].

    Returns (out [G, d], lse [G], mass [L // bs + 1]): the group-mean attention mass of
    every complete block, then of the tail (0 when L is a multiple of bs)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    G, d = q.shape
    if L is None:
        L = k.shape[0]
    assert k.shape[0] >= L and v.shape == k.shape
    out = np.zeros((G, d), dtype=np.float64)
    lse = np.zeros((G,), dtype=np.float64)
    mass = np.zeros((L // bs + 1,), dtype=np.float64)
    _check(_load().so_decode_block_mass(_p(q), d, G, d, _p(k), _p(v), d, L, bs, float(scale), _p(out), _p(lse),
                                        _p(mass)), "decode_block_mass")
    return out, lse, mass


def pool_cache(k, seqlens, bs: int, nb_max: int) -> np.ndarray:
    """Pooled keys of a batch: k [B, Hkv, cap, d] -> [B, Hkv, nb_max, d] (zero past each nc)."""
    k, seqlens = _u16(k), _i32(seqlens)
    B, H, cap, d = k.shape
    out = np.zeros((B, H, nb_max, d), dtype=np.float64)
    _check(_load().so_pool_cache(_p(k), H * cap * d, cap * d, d, _p(seqlens), B, H, d, bs, nb_max,
                                 _p(out)), "pool_cache")
    return out


def decode_step(q, k, v, seqlens, bs: int, budget: int, wq, wk, gate_scale: float, kpool,
                softmax_scale: float) -> dict:
    """One gated sparse decode step over a batch.

    q [B, Hq, d]; k, v [B, Hkv, cap, d]; wq, wk [Hkv, dg, d]; kpool [B, Hkv, nb_max, d] fp64."""
    q, k, v, wq, wk = _u16(q), _u16(k), _u16(v), _u16(wq), _u16(wk)
    seqlens, kpool = _i32(seqlens), _f64(kpool)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    dg = wq.shape[1]
    nb_max = kpool.shape[2]
    kmax = budget // bs
    scores = np.zeros((B, Hkv, nb_max), dtype=np.float64)
    idx = np.full((B, Hkv, max(kmax, 1)), -1, dtype=np.int32)
    n_sel = np.zeros((B, Hkv), dtype=np.int32)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    _check(_load().so_decode_step(_p(q), Hq * d, d, _p(k), _p(v), Hkv * cap * d, cap * d, d,
                                  _p(seqlens), B, Hq, Hkv, d, bs, int(budget), _p(wq), _p(wk), dg,
                                  float(gate_scale), _p(kpool), nb_max, float(softmax_scale),
                                  _p(scores), _p(idx), _p(n_sel), _p(out), _p(lse)), "decode_step")
    return {"scores": scores, "idx": idx[:, :, :kmax], "n_sel": n_sel, "out": out, "lse": lse}


def decode_step_per_head(q, k, v, seqlens, bs: int, budget: int, wq, wk, gate_scale: float, kpool,
                         softmax_scale: float) -> dict:
    """decode_step with per-query-head selection: scores, idx, n_sel per query head."""
    q, k, v, wq, wk = _u16(q), _u16(k), _u16(v), _u16(wq), _u16(wk)
    seqlens, kpool = _i32(seqlens), _f64(kpool)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    dg = wq.shape[1]
    nb_max = kpool.shape[2]
    kmax = budget // bs
    scores = np.zeros((B, Hq, nb_max), dtype=np.float64)
    idx = np.full((B, Hq, max(kmax, 1)), -1, dtype=np.int32)
    n_sel = np.zeros((B, Hq), dtype=np.int32)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    _check(_load().so_decode_step_per_head(_p(q), Hq * d, d, _p(k), _p(v), Hkv * cap * d, cap * d, d,
                                           _p(seqlens), B, Hq, Hkv, d, bs, int(budget), _p(wq), _p(wk), dg,
                                           float(gate_scale), _p(kpool), nb_max, float(softmax_scale),
                                           _p(scores), _p(idx), _p(n_sel), _p(out), _p(lse)), "decode_step_per_head")
    return {"scores": scores, "idx": idx[:, :, :kmax], "n_sel": n_sel, "out": out, "lse": lse}


def prefill_kmax_row(L: int, bs: int, keep_num: int, keep_den: int) -> int:
    nb = (L + bs - 1) // bs
    return max(1, min(nb, (nb * keep_num + keep_den - 1) // keep_den))


def prefill_gate(q, k, bs: int, wq, wk, gate_scale: float, keep_num: int, keep_den: int):
    """Gate of one prefill head: q, k [L, d]; returns (S [nb, nb], blocks [nb, kmax_row], counts [nb])."""
    q, k, wq, wk = _u16(q), _u16(k), _u16(wq), _u16(wk)
    L, d = q.shape
    dg = wq.shape[0]
    nb = (L + bs - 1) // bs
    kmax = prefill_kmax_row(L, bs, keep_num, keep_den)
    S = np.zeros((nb, nb), dtype=np.float64)
    blocks = np.full((nb, kmax), -1, dtype=np.int32)
    counts = np.zeros((nb,), dtype=np.int32)
    _check(_load().so_prefill_gate(_p(q), _p(k), d, L, d, bs, _p(wq), _p(wk), dg, float(gate_scale),
                                   keep_num, keep_den, _p(S), _p(blocks), _p(counts), kmax),
           "prefill_gate")
    return S, blocks, counts


def prefill_attention(q, k, v, bs: int, blocks, counts, scale: float, t_lo: int = 0,
                      t_hi: Optional[int] = None):
    """Block-sparse causal attention of one head for query tokens [t_lo, t_hi)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    blocks, counts = _i32(blocks), _i32(counts)
    L, d = q.shape
    t_hi = L if t_hi is None else t_hi
    out = np.zeros((t_hi - t_lo, d), dtype=np.float64)
    lse = np.zeros((t_hi - t_lo,), dtype=np.float64)
    _check(_load().so_prefill_attention(_p(q), _p(k), _p(v), d, L, d, bs, _p(blocks), _p(counts),
                                        blocks.shape[1], float(scale), t_lo, t_hi, _p(out), _p(lse)),
           "prefill_attention")
    return out, lse


def prefill_block_mass(q, k, bs: int, scale: float, i_lo: int = 0, i_hi: Optional[int] = None) -> np.ndarray:
    """Ground truth of one head's prefill: [i_hi - i_lo, nb] mean attention mass per (query block, key block)."""
    q, k = _u16(q), _u16(k)
    L, d = q.shape
    nb = (L + bs - 1) // bs
    i_hi = nb if i_hi is None else i_hi
    mass = np.zeros((i_hi - i_lo, nb), dtype=np.float64)
    _check(_load().so_prefill_block_mass(_p(q), _p(k), d, L, d, bs, float(scale), i_lo, i_hi, _p(mass)),
           "prefill_block_mass")
    return mass


def prefill(q, k, v, bs: int, wq, wk, gate_scale: float, keep_num: int, keep_den: int,
            scale: float, t_lo: int = 0, t_hi: Optional[int] = None) -> dict:
    """Gate + attention for every head of q, k, v [B, H, L, d]; query tokens [t_lo, t_hi)."""
    q, k, v, wq, wk = _u16(q), _u16(k), _u16(v), _u16(wq), _u16(wk)
    B, H, L, d = q.shape
    dg = wq.shape[1]
    t_hi = L if t_hi is None else t_hi
    nb = (L + bs - 1) // bs
    kmax = prefill_kmax_row(L, bs, keep_num, keep_den)
    blocks = np.full((B, H, nb, kmax), -1, dtype=np.int32)
    counts = np.zeros((B, H, nb), dtype=np.int32)
    out = np.zeros((B, H, t_hi - t_lo, d), dtype=np.float64)
    lse = np.zeros((B, H, t_hi - t_lo), dtype=np.float64)
    _check(_load().so_prefill(_p(q), _p(k), _p(v), B, H, L, d, bs, _p(wq), _p(wk), dg,
                              float(gate_scale), keep_num, keep_den, _p(blocks), _p(counts), kmax,
                              float(scale), t_lo, t_hi, _p(out), _p(lse)), "prefill")
    return {"blocks": blocks, "counts": counts, "out": out, "lse": lse}
