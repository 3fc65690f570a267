"""Pins of the oracle's sparse attention (steps D5 + D6) to things other than itself.

Softmax attention restricted to a token set has a plain definition, so the
pins are library routines (PyTorch's fp64 CPU scaled_dot_product_attention
and logsumexp, with a boolean mask built from the kept blocks), closed forms
and invariants.  Sources: "SeerAttention-R: Sparse Attention Adaptation for
Long Reasoning", abstract (sparse decoding over selected blocks); "SeerAttention:
Learning Intrinsic Sparse Attention in Your LLMs", abstract v2 (unselected
blocks are sparse, i.e. get no weight).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def bf16(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)


def token_mask(L, bs, idx):
    nc = L // bs
    m = torch.zeros(L, dtype=torch.bool)
    for j in idx:
        m[j * bs:(j + 1) * bs] = True
    m[nc * bs:L] = True
    return m


def sdpa_reference(q_bits, k_bits, v_bits, mask, scale):
    q = widen(q_bits)[None, :, None, :]            # [1, G, 1, d]
    k = widen(k_bits)[None, None].expand(1, q.shape[1], -1, -1)
    v = widen(v_bits)[None, None].expand(1, q.shape[1], -1, -1)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None, None, :], scale=scale)
    logits = (q @ k.transpose(-1, -2))[0, :, 0, :] * scale
    logits = logits.masked_fill(~mask[None, :], -math.inf)
    return out[0, :, 0, :].numpy(), torch.logsumexp(logits, dim=-1).numpy()


def rand_case(G, d, L, seed):
    g = torch.Generator().manual_seed(seed)
    q = bf16(torch.randn(G, d, generator=g))
    k = bf16(torch.randn(L, d, generator=g))
    v = bf16(torch.randn(L, d, generator=g))
    return q, k, v


@pytest.mark.parametrize("G,d,L,bs", [(4, 64, 300, 64), (1, 128, 256, 128), (8, 64, 1000, 64), (2, 32, 7, 64)])
def test_all_blocks_selected_equals_dense_attention(G, d, L, bs):
    """Pin: every block selected -> plain dense softmax attention."""
    q, k, v = rand_case(G, d, L, seed=G * 1000 + L)
    scale = 1.0 / math.sqrt(d)
    idx = np.arange(L // bs, dtype=np.int32)
    out, lse, _ = oracle.sparse_attention(q, k, v, bs, idx, scale)
    ref_out, ref_lse = sdpa_reference(q, k, v, torch.ones(L, dtype=torch.bool), scale)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_sparse_equals_masked_dense(seed):
    """Brute force: sparse attention == dense attention with -inf outside the kept blocks + tail."""
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([64, 128]))
    L = int(rng.integers(bs, 8 * bs + bs))
    nc = L // bs
    G, d = int(rng.choice([1, 4, 8])), int(rng.choice([32, 64, 128]))
    q, k, v = rand_case(G, d, L, seed=100 + seed)
    idx = np.sort(rng.choice(nc, size=int(rng.integers(0, nc + 1)), replace=False)).astype(np.int32)
    scale = float(rng.uniform(0.05, 0.3))
    mask = token_mask(L, bs, idx)
    if not mask.any():
        pytest.skip("empty token set covered separately")
    out, lse, w = oracle.sparse_attention(q, k, v, bs, idx, scale, want_weights=True)
    ref_out, ref_lse = sdpa_reference(q, k, v, mask, scale)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    # pin: softmax weights sum to one, and vanish outside T
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w[:, ~mask.numpy()] == 0.0)


def test_single_token_returns_its_value():
    """|T| = 1: the output is that token's value row; lse is its logit."""
    q, k, v = rand_case(3, 64, 1, seed=7)
    out, lse, _ = oracle.sparse_attention(q, k, v, 64, np.zeros(0, np.int32), 0.125)
    np.testing.assert_array_equal(out, np.broadcast_to(widen(v)[0].numpy(), out.shape))
    z = (widen(q) @ widen(k)[0]).numpy() * 0.125
    np.testing.assert_allclose(lse, z, rtol=0, atol=1e-14)


def test_equal_keys_give_mean_of_values():
    """All keys in T equal -> uniform weights -> o = mean of V over T (tail included)."""
    L, bs, d = 64 * 5 + 9, 64, 64
    g = torch.Generator().manual_seed(3)
    q = bf16(torch.randn(4, d, generator=g))
    row = torch.randn(d, generator=g)
    k = bf16(row.expand(L, d).clone())
    v = bf16(torch.randn(L, d, generator=g))
    idx = np.array([1, 3], dtype=np.int32)
    out, lse, _ = oracle.sparse_attention(q, k, v, bs, idx, 0.125)
    mask = token_mask(L, bs, idx)
    expect = widen(v)[mask].mean(dim=0).numpy()
    np.testing.assert_allclose(out, np.broadcast_to(expect, out.shape), rtol=0, atol=1e-12)
    z = (widen(q) @ widen(k)[0]).numpy() * 0.125
    np.testing.assert_allclose(lse, z + math.log(int(mask.sum())), rtol=0, atol=1e-12)


def test_equal_values_give_that_value():
    L, bs, d = 512, 128, 128
    g = torch.Generator().manual_seed(4)
    q = bf16(torch.randn(2, d, generator=g))
    k = bf16(torch.randn(L, d, generator=g))
    vrow = torch.randn(d, generator=g)
    v = bf16(vrow.expand(L, d).clone())
    out, _, _ = oracle.sparse_attention(q, k, v, bs, np.array([0, 2], np.int32), 1 / math.sqrt(d))
    np.testing.assert_allclose(out, np.broadcast_to(widen(v)[0].numpy(), out.shape), rtol=0, atol=1e-12)


def test_empty_token_set():
    """k = 0 with no tail: nothing to attend -> zeros, lse = -inf (documented convention)."""
    q, k, v = rand_case(2, 64, 128, seed=5)
    out, lse, _ = oracle.sparse_attention(q, k, v, 64, np.zeros(0, np.int32), 0.125)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def test_tail_only():
    """Budget below one block: only the incomplete tail [nc*bs, L) is attended."""
    L, bs = 64 * 3 + 5, 64
    q, k, v = rand_case(4, 64, L, seed=6)
    out, _, _ = oracle.sparse_attention(q, k, v, bs, np.zeros(0, np.int32), 0.125)
    ref, _ = sdpa_reference(q, k[192:], v[192:], torch.ones(5, dtype=torch.bool), 0.125)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_rejects_unsorted_or_out_of_range_blocks():
    q, k, v = rand_case(1, 64, 256, seed=8)
    for bad in ([2, 1], [0, 0], [4], [-1]):
        with pytest.raises(ValueError):
            oracle.sparse_attention(q, k, v, 64, np.array(bad, np.int32), 0.125)
